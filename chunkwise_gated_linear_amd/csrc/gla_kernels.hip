// Device kernels of the chunkwise gated linear attention forward, gfx950.
//
// Method (page "fla/ops/gla/fused_chunk.py"): per sequence and head, a K x V
// fp32 state S is carried across chunks of 64 tokens.  Inside a chunk, with
// E_s = exp(g_s) per key and running products P_i = prod_{s<=i} E_s,
// a = P_last, R_j = prod_{s>j} E_s (the page's exp(G), exp(G_last) and
// exp(G_last - G) of prepare_qg_kg / fused_chunk_gla_fwd_kernel, formed as
// products of exp(g) so that one exponential per element suffices):
//
//   qc_i = scale * q_i * P_i / a       kc_j = k_j * R_j
//   A_ij = qc_i . kc_j  for j <= i     (fwd_inner_chunk's masked gated scores)
//   S'   = diag(a) S                    (decay of the carried state)
//   o_i  = sum_j A_ij v_j + qc_i S'     (in-chunk term + inter-chunk term)
//   S    = S' + kc^T v                  (state after the chunk)
//
// qc_i S' = scale q_i diag(P_i) S, so the inter-chunk term uses the state
// before the chunk exactly as fused_chunk_gla_fwd_kernel does, and the
// in-chunk term weights key j by exp(G_i - G_j) as fwd_inner_chunk does.
//
// Kernels:
//   gla_chunk_local   walks one state segment (R chunks) from a zero state and
//                     writes its summary: diag-decay product and K x V state.
//   gla_state_scan    per state element, folds the segment summaries of each
//                     sequence into the start state of every segment.
//   gla_chunk_output  walks one segment from its start state, writes o and,
//                     for the last segment, the final state.
// With one segment per sequence only gla_chunk_output runs.
//
// Precision: the bf16 instantiation feeds MFMA v_mfma_f32_16x16x32_bf16 with
// operands split into bf16 hi + lo parts (x = hi + lo to ~16 bits), using
// hi*hi + lo*hi + hi*lo for products of two computed operands and hi*x + lo*x
// against the exact bf16 inputs v.  Accumulation is fp32.  The fp32
// instantiation uses v_mfma_f32_16x16x4_f32.
//
// Workgroup: 256 threads = 4 waves; one workgroup owns one (segment, head,
// 64-column slice of V).  Wave w owns value columns [16w, 16w+16) of the
// slice; its lanes hold the KD x 16 state block in MFMA accumulator layout
// (lane l: column l%16, rows 16*kt + 4*(l/16) + r).
//
// Shapes: a launch covers one key block of K <= KD keys (the instantiation's
// width KD; keys K..KD-1 are zero padding: g = 0, q = k = 0, so they add
// nothing and decay by exp(0) = 1) and value columns v0.. of each slice below V
// (columns past V read as zero and are never stored).  With two key blocks the
// first writes its fp32 partial output to o_part and the second adds it.
#include "gla_internal.h"
#include "gla_device.h"

#include <cstdlib>
#include <type_traits>

namespace gla {
namespace {

using namespace dev;

// ---------------------------------------------------------------- LDS plan
template <bool BF, int KD, bool OUT>
struct Lds {
  static constexpr int ES = BF ? 2 : 4;                 // element bytes of operands
  static constexpr int NS = BF ? 2 : 1;                 // hi/lo planes
  static constexpr int QROW = KD * ES + 16;             // [token][k] rows, padded
  static constexpr int TROW = C * ES + 16;              // [k or n or i][token] rows
  static constexpr int OROW = VT * ES + 16;             // output staging rows
  static constexpr int NQ = KD / 4;                     // prologue column quads
  static constexpr int NG = kThreads / NQ;              // prologue row groups
  static constexpr int Q_PLANE = C * QROW;
  static constexpr int KT_PLANE = KD * TROW;
  static constexpr int A_PLANE = C * TROW;
  // offsets
  static constexpr int oQ = 0;                                   // qc  [C][K]   (OUT)
  static constexpr int oK = oQ + (OUT ? NS * Q_PLANE : 0);        // kc  [C][K]   (OUT)
  static constexpr int oKT = oK + (OUT ? NS * Q_PLANE : 0);       // kc^T [K][C]
  static constexpr int oVT = oKT + NS * KT_PLANE;                // v^T [VT][C]
  static constexpr int oA = oVT + VT * TROW;                     // A   [C][C]   (OUT)
  static constexpr int oO = oA + (OUT ? NS * A_PLANE : 0);        // o   [C][VT]  (OUT)
  static constexpr int oDec = oO + (OUT ? C * OROW : 0);          // a   [K] fp32
  static constexpr int oTot = oDec + KD * 4;                     // group products [NG][K]
  static constexpr int oBad = oTot + NG * KD * 4;                 // a chunk needs the exact path (OUT)
  static constexpr int BYTES = oBad + 16;
};

// P1 tiles (i-tile, j-tile) per wave: the 10 lower-triangular 16x16 tiles of the 64x64 score block.
__constant__ const int8_t kP1[4][3][2] = {
    {{0, 0}, {1, 0}, {1, 1}},
    {{2, 0}, {2, 1}, {2, 2}},
    {{3, 0}, {3, 1}, {-1, -1}},
    {{3, 2}, {3, 3}, {-1, -1}},
};

// ---------------------------------------------------------------- the chunk walker
// OUT = false: gla_chunk_local (segment summary).  OUT = true: gla_chunk_output.
// GH: one decay per value head and token (g [B,T,HV]) instead of one per key.
template <bool OUT, bool BF, int KD, bool GH>
__device__ __forceinline__ void walk(const WalkParams &p, char *smem) {
  using L = Lds<BF, KD, OUT>;
  constexpr int ES = L::ES;
  constexpr int NQ = L::NQ, NG = L::NG, RPG = C / NG;   // prologue mapping
  constexpr int NKT = KD / 16;                            // 16-row k tiles
  constexpr int KB = BF ? 32 : 16;                        // contraction block of one MFMA step
  constexpr int NKB = KD / KB;
  constexpr int NJB = C / KB;
  static_assert(NG * NQ == kThreads && RPG * NG == C && RPG >= 1, "prologue mapping");
  static_assert(KD % KB == 0, "K must be a multiple of the contraction block");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  // ---- which (segment, head, value slice) this workgroup owns; the value
  // slices of one unit sit 8 workgroup ids apart so they land on one XCD.
  const int NV = (p.V + VT - 1) / VT;
  const int b = blockIdx.x;
  const int grp = b / (8 * NV), rem = b - grp * (8 * NV);
  const int vt = rem >> 3;
  const int unit = grp * 8 + (rem & 7);
  if (unit >= p.units) return;
  const int seg = unit / p.HV, h = unit - seg * p.HV;  // h: value head
  SegInfo si;
  if (!locate(p, seg, si)) return;
  if (!OUT && si.s >= si.nseg - 1) return;  // the last segment's summary is never used
  const int nchunks = (si.len + C - 1) / C;
  // the sequence's nseg = max(1, ceil(nchunks / R)) segments share its chunks
  // evenly: ceil(nchunks / nseg) <= R each, none empty
  const int seg_len = (nchunks + si.nseg - 1) / si.nseg;
  const int c_begin = si.s * seg_len;
  const int c_end = min(c_begin + seg_len, nchunks);
  const int v0 = vt * VT;
  const int H = p.HV;                   // value heads: v, o, g, states
  const int nkeys = p.K;                // real keys of this block (<= KD)
  const size_t rowK = (size_t)p.H * p.Kmem;  // element stride between tokens, q/k
  const size_t rowV = (size_t)H * p.V;       // element stride between tokens, v/o
  const size_t headK = (size_t)(h / p.G) * p.Kmem + p.koff;  // first key of the block, key head of h
  // g: a decay per key [.., HV, Kmem] or one per value head [.., HV]
  const size_t rowG = GH ? (size_t)H : (size_t)H * p.Kmem;
  const size_t headG = GH ? (size_t)h : (size_t)h * p.Kmem + p.koff;

  // ---- state block of this lane: S[16kt + 4lg + r][v0 + 16wave + l16]
  f32x4_t S[NKT];
  const int scol = v0 + 16 * wave + l16;
  const bool col_ok = scol < p.V;
  {
    // h0 rows are [Kmem] wide (this block's rows start at koff), start states [K]
    const float *src = nullptr;
    if (OUT) {
      if (si.s == 0) {
        if (p.h0) src = p.h0 + (((size_t)si.n * H + h) * p.Kmem + p.koff) * p.V;
      } else {
        src = p.seg_state + ((size_t)(si.first + si.s - 1) * H + h) * nkeys * p.V;
      }
    }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * kt + 4 * lg + r;
        S[kt][r] = (src && col_ok && row < nkeys) ? src[(size_t)row * p.V + scol] : 0.f;
      }
  }

  // zero the score block once: tiles above the diagonal are read by the
  // 32-wide contraction steps but never written.
  if (OUT) {
    for (int i = tid; i < L::NS * L::A_PLANE / 16; i += kThreads)
      lds_st<u32x4_t>(smem + L::oA, i * 16, u32x4_t{0, 0, 0, 0});
  }

  // ---- prologue register mapping: rows [rg*RPG, rg*RPG+RPG), columns 4cq..4cq+3
  const int cq = tid % NQ, rg = tid / NQ;
  // v mapping: rows 4vg..4vg+3, columns 4vq..4vq+3 of the slice
  const int vq = tid & 15, vg = tid >> 4;

  using QReg = typename std::conditional<BF, u32x2_t, f32x4_t>::type;
  f32x4_t rg_g[RPG];
  QReg rg_q[RPG], rg_k[RPG], rg_v[4];

  const bool key_ok = 4 * cq < nkeys;        // this thread's key quad is a real key
  const bool vcol_ok = v0 + 4 * vq < p.V;  // this thread's v column quad exists
  auto load_chunk = [&](int c) {
    const size_t t0 = (size_t)si.bos + (size_t)c * C;
    const int valid = min(C, si.len - c * C);
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
      const int row = rg * RPG + r;
      const bool ok = row < valid && key_ok;
      const size_t off = (t0 + row) * rowK + headK + 4 * cq;
      if constexpr (GH) {  // one decay for every key of the row
        const float x = ok ? p.g[(t0 + row) * rowG + headG] : 0.f;
        rg_g[r] = f32x4_t{x, x, x, x};
      } else {
        rg_g[r] = ok ? *reinterpret_cast<const f32x4_t *>(p.g + (t0 + row) * rowG + headG + 4 * cq) : f32x4_t{0, 0, 0, 0};
      }
      if constexpr (BF) {
        rg_k[r] = ok ? *reinterpret_cast<const u32x2_t *>((const uint16_t *)p.k + off) : u32x2_t{0, 0};
        if (OUT) rg_q[r] = ok ? *reinterpret_cast<const u32x2_t *>((const uint16_t *)p.q + off) : u32x2_t{0, 0};
      } else {
        rg_k[r] = ok ? *reinterpret_cast<const f32x4_t *>((const float *)p.k + off) : f32x4_t{0, 0, 0, 0};
        if (OUT) rg_q[r] = ok ? *reinterpret_cast<const f32x4_t *>((const float *)p.q + off) : f32x4_t{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * vg + r;
      const bool ok = row < valid && vcol_ok;
      const size_t off = (t0 + row) * rowV + (size_t)h * p.V + v0 + 4 * vq;
      if constexpr (BF)
        rg_v[r] = ok ? *reinterpret_cast<const u32x2_t *>((const uint16_t *)p.v + off) : u32x2_t{0, 0};
      else
        rg_v[r] = ok ? *reinterpret_cast<const f32x4_t *>((const float *)p.v + off) : f32x4_t{0, 0, 0, 0};
    }
  };

  float seg_decay[4] = {1.f, 1.f, 1.f, 1.f};  // product of chunk decays (summary mode)
  bool seg_bad = false;  // some key of a chunk decayed by more than kMinChunkDecay (OUT)
  const float scale = p.scale;
  if (OUT && tid == 0) lds_st<int>(smem + L::oBad, 0, 0);

  if (c_begin < c_end) load_chunk(c_begin);

  for (int c = c_begin; c < c_end; ++c) {
    // ================= prologue: decays, gated operands -> LDS
    float E[RPG][4];
#pragma unroll
    for (int r = 0; r < RPG; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) E[r][j] = __expf(rg_g[r][j]);
    float Pl[RPG][4], Rl[RPG][4];  // inclusive prefix / exclusive suffix products in the group
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      Pl[0][j] = E[0][j];
#pragma unroll
      for (int r = 1; r < RPG; ++r) Pl[r][j] = Pl[r - 1][j] * E[r][j];
      Rl[RPG - 1][j] = 1.f;
#pragma unroll
      for (int r = RPG - 2; r >= 0; --r) Rl[r][j] = Rl[r + 1][j] * E[r + 1][j];
    }
    lds_st<f32x4_t>(smem + L::oTot, (rg * KD + 4 * cq) * 4,
                    f32x4_t{Pl[RPG - 1][0], Pl[RPG - 1][1], Pl[RPG - 1][2], Pl[RPG - 1][3]});
    __syncthreads();
    float pre[4] = {1.f, 1.f, 1.f, 1.f}, suf[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const f32x4_t t = lds_ld<f32x4_t>(smem + L::oTot, (gi * KD + 4 * cq) * 4);
      if (gi < rg) {
#pragma unroll
        for (int j = 0; j < 4; ++j) pre[j] *= t[j];
      } else if (gi > rg) {
#pragma unroll
        for (int j = 0; j < 4; ++j) suf[j] *= t[j];
      }
    }
    float dec[4], fq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dec[j] = pre[j] * Pl[RPG - 1][j] * suf[j];   // a = product over the whole chunk
      fq[j] = OUT ? scale * pre[j] / dec[j] : 0.f;
      // beyond this decay scale q exp(G - G_last) overflows: the segment's
      // outputs are then re-evaluated token by token
      if (OUT) seg_bad = seg_bad || dec[j] < kMinChunkDecay;
    }
    if (rg == 0) {
      lds_st<f32x4_t>(smem + L::oDec, 16 * cq, f32x4_t{dec[0], dec[1], dec[2], dec[3]});
      if (!OUT) {
#pragma unroll
        for (int j = 0; j < 4; ++j) seg_decay[j] *= dec[j];
      }
    }

    // gated operands: qc, kc row-major (OUT), kc transposed
    using KSplit = typename std::conditional<BF, u32x2_t, f32x4_t>::type;
    KSplit kt_hi[RPG], kt_lo[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
      const int row = rg * RPG + r;
      float kc[4], qc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float kk, qq = 0.f;
        if constexpr (BF) {
          kk = (j & 1) ? bf_hi(rg_k[r][j >> 1]) : bf_lo(rg_k[r][j >> 1]);
          if (OUT) qq = (j & 1) ? bf_hi(rg_q[r][j >> 1]) : bf_lo(rg_q[r][j >> 1]);
        } else {
          kk = rg_k[r][j];
          if (OUT) qq = rg_q[r][j];
        }
        kc[j] = kk * (Rl[r][j] * suf[j]);
        qc[j] = qq * (Pl[r][j] * fq[j]);
      }
      if constexpr (BF) {
        const int off = row * L::QROW + kperm_bf(4 * cq) * 2;
        split4_sub(kc, kt_hi[r], kt_lo[r]);
        if (OUT) {
          u32x2_t qh, ql;
          split4_sub(qc, qh, ql);
          lds_st<u32x2_t>(smem + L::oQ, off, qh);
          lds_st<u32x2_t>(smem + L::oQ + L::Q_PLANE, off, ql);
          lds_st<u32x2_t>(smem + L::oK, off, kt_hi[r]);
          lds_st<u32x2_t>(smem + L::oK + L::Q_PLANE, off, kt_lo[r]);
        }
      } else {
        kt_hi[r] = f32x4_t{kc[0], kc[1], kc[2], kc[3]};
        if (OUT) {
          const int off = row * L::QROW + 16 * cq;
          lds_st<f32x4_t>(smem + L::oQ, off, f32x4_t{qc[0], qc[1], qc[2], qc[3]});
          lds_st<f32x4_t>(smem + L::oK, off, kt_hi[r]);
        }
      }
    }
    // kc^T [k][token]: this thread's RPG consecutive tokens of column 4cq+j are contiguous
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = (4 * cq + j) * L::TROW + rg * RPG * ES;
      if constexpr (BF) {
#pragma unroll
        for (int plane = 0; plane < 2; ++plane) {
          const KSplit *src = plane ? kt_lo : kt_hi;
          char *base = smem + L::oKT + plane * L::KT_PLANE;
          uint16_t e[RPG];
#pragma unroll
          for (int r = 0; r < RPG; ++r)
            e[r] = (uint16_t)((j & 1) ? (src[r][j >> 1] >> 16) : (src[r][j >> 1] & 0xffffu));
          if constexpr (RPG == 1) {
            lds_st<uint16_t>(base, off, e[0]);
          } else {
            uint32_t w[RPG / 2];
#pragma unroll
            for (int m = 0; m < RPG / 2; ++m) w[m] = (uint32_t)e[2 * m] | ((uint32_t)e[2 * m + 1] << 16);
            if constexpr (RPG == 2) lds_st<uint32_t>(base, off, w[0]);
            else if constexpr (RPG == 4) lds_st<u32x2_t>(base, off, u32x2_t{w[0], w[1]});
            else {
#pragma unroll
              for (int m = 0; m < RPG / 8; ++m)
                lds_st<u32x4_t>(base, off + 16 * m, u32x4_t{w[4 * m], w[4 * m + 1], w[4 * m + 2], w[4 * m + 3]});
            }
          }
        }
      } else {
        char *base = smem + L::oKT;
        if constexpr (RPG == 1) {
          lds_st<float>(base, off, kt_hi[0][j]);
        } else if constexpr (RPG == 2) {
          typedef float f32x2_t __attribute__((ext_vector_type(2)));
          lds_st<f32x2_t>(base, off, f32x2_t{kt_hi[0][j], kt_hi[1][j]});
        } else {
#pragma unroll
          for (int m = 0; m < RPG / 4; ++m)
            lds_st<f32x4_t>(base, off + 16 * m,
                            f32x4_t{kt_hi[4 * m][j], kt_hi[4 * m + 1][j], kt_hi[4 * m + 2][j], kt_hi[4 * m + 3][j]});
        }
      }
    }
    // v^T: [n][token]
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (BF) {
        uint32_t w0, w1;
        const uint32_t a0 = rg_v[0][j >> 1], a1 = rg_v[1][j >> 1], a2 = rg_v[2][j >> 1], a3 = rg_v[3][j >> 1];
        if (j & 1) {
          w0 = (a0 >> 16) | (a1 & 0xffff0000u);
          w1 = (a2 >> 16) | (a3 & 0xffff0000u);
        } else {
          w0 = (a0 & 0xffffu) | (a1 << 16);
          w1 = (a2 & 0xffffu) | (a3 << 16);
        }
        lds_st<u32x2_t>(smem + L::oVT, (4 * vq + j) * L::TROW + (4 * vg) * 2, u32x2_t{w0, w1});
      } else {
        lds_st<f32x4_t>(smem + L::oVT, (4 * vq + j) * L::TROW + (4 * vg) * 4,
                        f32x4_t{rg_v[0][j], rg_v[1][j], rg_v[2][j], rg_v[3][j]});
      }
    }
    // next chunk's loads go out now and land while this chunk computes
    if (c + 1 < c_end) load_chunk(c + 1);
    __syncthreads();

    // ================= MFMA phase
    if constexpr (OUT) {
      // ---- P1: A^T tiles = kc qc^T, masked j <= i, split, -> LDS A[i][j]
#pragma unroll
      for (int tix = 0; tix < 3; ++tix) {
        const int it = kP1[wave][tix][0], jt = kP1[wave][tix][1];
        if (it < 0) continue;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        const int arow = 16 * jt + l16, brow = 16 * it + l16;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          if constexpr (BF) {
            const int off_a = arow * L::QROW + (kb * 32 + 8 * lg) * 2;
            const int off_b = brow * L::QROW + (kb * 32 + 8 * lg) * 2;
            const u32x4_t ah = lds_ld<u32x4_t>(smem + L::oK, off_a);
            const u32x4_t al = lds_ld<u32x4_t>(smem + L::oK + L::Q_PLANE, off_a);
            const u32x4_t bh = lds_ld<u32x4_t>(smem + L::oQ, off_b);
            const u32x4_t bl = lds_ld<u32x4_t>(smem + L::oQ + L::Q_PLANE, off_b);
            acc = mfma_bf(al, bh, acc);
            acc = mfma_bf(ah, bl, acc);
            acc = mfma_bf(ah, bh, acc);
          } else {
            const f32x4_t a4 = lds_ld<f32x4_t>(smem + L::oK, arow * L::QROW + (kb * 16 + 4 * lg) * 4);
            const f32x4_t b4 = lds_ld<f32x4_t>(smem + L::oQ, brow * L::QROW + (kb * 16 + 4 * lg) * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc = mfma_f32(a4[r], b4[r], acc);
          }
        }
        // lane: i = 16it + l16, j = 16jt + 4lg + r
        const int i = 16 * it + l16;
        float av[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) av[r] = (16 * jt + 4 * lg + r <= i) ? acc[r] : 0.f;
        const int off = i * L::TROW + (16 * jt + 4 * lg) * ES;
        if constexpr (BF) {
          u32x2_t hi, lo;
          split4_sub(av, hi, lo);
          lds_st<u32x2_t>(smem + L::oA, off, hi);
          lds_st<u32x2_t>(smem + L::oA + L::A_PLANE, off, lo);
        } else {
          lds_st<f32x4_t>(smem + L::oA, off, f32x4_t{av[0], av[1], av[2], av[3]});
        }
      }
      __syncthreads();
    }

    // ---- decay the carried state: S' = diag(a) S
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const f32x4_t a4 = lds_ld<f32x4_t>(smem + L::oDec, (16 * kt + 4 * lg) * 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) S[kt][r] *= a4[r];
    }

    // v^T fragments of this wave's 16 columns (B operand of P2 and P4)
    using VFrag = typename std::conditional<BF, u32x4_t, f32x4_t>::type;
    VFrag vf[NJB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
      const int off = (16 * wave + l16) * L::TROW + (jb * KB + (BF ? 8 : 4) * lg) * ES;
      vf[jb] = lds_ld<VFrag>(smem + L::oVT, off);
    }

    if constexpr (OUT) {
      f32x4_t o[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) o[it] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // ---- P2: o += A v over the causal j-blocks
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int jbmax = (16 * it + 15) / KB;
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
          if (jb > jbmax) continue;
          const int off = (16 * it + l16) * L::TROW + (jb * KB + (BF ? 8 : 4) * lg) * ES;
          if constexpr (BF) {
            const u32x4_t ah = lds_ld<u32x4_t>(smem + L::oA, off);
            const u32x4_t al = lds_ld<u32x4_t>(smem + L::oA + L::A_PLANE, off);
            o[it] = mfma_bf(al, vf[jb], o[it]);
            o[it] = mfma_bf(ah, vf[jb], o[it]);
          } else {
            const f32x4_t a4 = lds_ld<f32x4_t>(smem + L::oA, off);
#pragma unroll
            for (int r = 0; r < 4; ++r) o[it] = mfma_f32(a4[r], vf[jb][r], o[it]);
          }
        }
      }
      // ---- P3: o += qc S'   (S' from this lane's accumulators)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if constexpr (BF) {
          const float s8[8] = {S[2 * kb][0], S[2 * kb][1], S[2 * kb][2], S[2 * kb][3],
                               S[2 * kb + 1][0], S[2 * kb + 1][1], S[2 * kb + 1][2], S[2 * kb + 1][3]};
          u32x2_t h0, l0, h1, l1;
          split4_sub(s8, h0, l0);  // the state stays live
          split4_sub(s8 + 4, h1, l1);
          const u32x4_t sh = {h0[0], h0[1], h1[0], h1[1]};
          const u32x4_t sl = {l0[0], l0[1], l1[0], l1[1]};
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const int off = (16 * it + l16) * L::QROW + (kb * 32 + 8 * lg) * 2;
            const u32x4_t qh = lds_ld<u32x4_t>(smem + L::oQ, off);
            const u32x4_t ql = lds_ld<u32x4_t>(smem + L::oQ + L::Q_PLANE, off);
            o[it] = mfma_bf(ql, sh, o[it]);
            o[it] = mfma_bf(qh, sl, o[it]);
            o[it] = mfma_bf(qh, sh, o[it]);
          }
        } else {
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const f32x4_t q4 = lds_ld<f32x4_t>(smem + L::oQ, (16 * it + l16) * L::QROW + (kb * 16 + 4 * lg) * 4);
#pragma unroll
            for (int r = 0; r < 4; ++r) o[it] = mfma_f32(q4[r], S[kb][r], o[it]);
          }
        }
      }
      // ---- key blocks: add the other block's fp32 partial output, or write this
      // block's partial instead of o (rows 16it + 4lg + r, column scol)
      if (p.o_add != nullptr || p.o_part != nullptr) {
        const int valid = min(C, si.len - c * C);
        const size_t t0 = (size_t)si.bos + (size_t)c * C;
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * it + 4 * lg + r;
            if (row < valid && col_ok) {
              const size_t idx = (t0 + row) * rowV + (size_t)h * p.V + scol;
              if (p.o_add != nullptr) o[it][r] += p.o_add[idx];
              else p.o_part[idx] = o[it][r];
            }
          }
      }
      // ---- stage o (rows 16it + 4lg + r, column 16wave + l16) for coalesced stores
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int off = (16 * it + 4 * lg + r) * L::OROW + (16 * wave + l16) * ES;
          if constexpr (BF)
            lds_st<__bf16>(smem + L::oO, off, (__bf16)o[it][r]);
          else
            lds_st<float>(smem + L::oO, off, o[it][r]);
        }
    }

    // ---- P4: S = S' + kc^T v
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const int off = (16 * kt + l16) * L::TROW + (jb * KB + (BF ? 8 : 4) * lg) * ES;
        if constexpr (BF) {
          const u32x4_t ah = lds_ld<u32x4_t>(smem + L::oKT, off);
          const u32x4_t al = lds_ld<u32x4_t>(smem + L::oKT + L::KT_PLANE, off);
          S[kt] = mfma_bf(al, vf[jb], S[kt]);
          S[kt] = mfma_bf(ah, vf[jb], S[kt]);
        } else {
          const f32x4_t a4 = lds_ld<f32x4_t>(smem + L::oKT, off);
#pragma unroll
          for (int r = 0; r < 4; ++r) S[kt] = mfma_f32(a4[r], vf[jb][r], S[kt]);
        }
      }
    }
    __syncthreads();

    if (OUT && p.o_part == nullptr) {
      // ---- coalesced output stores: 16-byte pieces of the staged tile (a piece
      // holds 16 / ES columns, all below V or all past it)
      const int valid = min(C, si.len - c * C);
      const size_t t0 = (size_t)si.bos + (size_t)c * C;
      constexpr int PIECES_PER_ROW = VT * ES / 16;
      for (int pc = tid; pc < C * PIECES_PER_ROW; pc += kThreads) {
        const int row = pc / PIECES_PER_ROW, piece = pc - row * PIECES_PER_ROW;
        if (row < valid && v0 + piece * (16 / ES) < p.V) {
          const u32x4_t val = lds_ld<u32x4_t>(smem + L::oO, row * L::OROW + piece * 16);
          char *dst = reinterpret_cast<char *>(p.o) +
                      (((t0 + row) * rowV + (size_t)h * p.V + v0) * ES) + piece * 16;
          *reinterpret_cast<u32x4_t *>(dst) = val;
        }
      }
    }
  }

  // ================= results of the segment
  if constexpr (OUT) {
    if (seg_bad) lds_st<int>(smem + L::oBad, 0, 1);
    __syncthreads();  // also orders the chunk loop's output stores before a rewrite
    if (__builtin_amdgcn_readfirstlane(lds_ld<int>(smem + L::oBad, 0)) != 0)
      exact_segment<KD, BF, true>(p, si, h, v0, VT, c_begin, c_end, wave, vt, nullptr);
  }
  // (rows of padded keys and columns past V are not stored)
  float *dst = nullptr;
  if constexpr (OUT) {
    if (p.ht != nullptr && si.s == si.nseg - 1) dst = p.ht + (((size_t)si.n * H + h) * p.Kmem + p.koff) * p.V;
  } else {
    dst = p.seg_state + ((size_t)(si.first + si.s) * H + h) * nkeys * p.V;
  }
  if (dst != nullptr && col_ok) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * kt + 4 * lg + r;
        if (row < nkeys) dst[(size_t)row * p.V + scol] = S[kt][r];
      }
  }
  if (!OUT && vt == 0 && rg == 0 && key_ok) {
    *reinterpret_cast<f32x4_t *>(p.seg_decay + ((size_t)(si.first + si.s) * H + h) * nkeys + 4 * cq) =
        f32x4_t{seg_decay[0], seg_decay[1], seg_decay[2], seg_decay[3]};
  }
}

template <bool BF, int KD, bool GH>
__global__ __launch_bounds__(kThreads, 1) void gla_chunk_local(WalkParams p) {
  __shared__ __attribute__((aligned(16))) char smem[Lds<BF, KD, false>::BYTES];
  walk<false, BF, KD, GH>(p, smem);
}

template <bool BF, int KD, bool GH>
__global__ __launch_bounds__(kThreads, 1) void gla_chunk_output(WalkParams p) {
  __shared__ __attribute__((aligned(16))) char smem[Lds<BF, KD, true>::BYTES];
  walk<true, BF, KD, GH>(p, smem);
}

// ---------------------------------------------------------------- state scan
// One thread per 4 consecutive state elements of one (sequence, head) of the
// key block: start(0) = h0 or 0, start(s+1) = diag(decay_s) start(s) +
// summary_s; the start state of segment s+1 overwrites the summary slot of
// segment s.  A 1-D grid: block b covers (sequence, head) b / per_state, and
// 1024 elements of its K x V state.
__global__ __launch_bounds__(256) void gla_state_scan(WalkParams p, int per_state) {
  const long long pair = blockIdx.x / per_state;
  const int eb = (int)(blockIdx.x - pair * per_state);
  const int n = (int)(pair / p.HV), h = (int)(pair - (long long)n * p.HV);
  const int e4 = eb * 256 + threadIdx.x;
  const int KV4 = p.K * p.V / 4;  // V is a multiple of 16: a quad never crosses a row
  if (n >= p.N || e4 >= KV4) return;
  int first, nseg;
  if (p.seg_base == nullptr) {
    first = n * p.P;
    nseg = p.P;
  } else {
    first = p.seg_base[n];
    nseg = p.seg_base[n + 1] - first;
  }
  if (nseg <= 1) return;
  const int krow = (4 * e4) / p.V, col = 4 * e4 - krow * p.V;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
  if (p.h0)
    s = *reinterpret_cast<const f32x4_t *>(p.h0 + (((size_t)n * p.HV + h) * p.Kmem + p.koff + krow) * p.V + col);
  for (int j = 0; j + 1 < nseg; ++j) {
    const size_t slot = (size_t)(first + j) * p.HV + h;
    const float a = p.seg_decay[slot * p.K + krow];
    f32x4_t *cell = reinterpret_cast<f32x4_t *>(p.seg_state + slot * p.K * p.V) + e4;
    const f32x4_t u = *cell;
    s = a * s + u;
    *cell = s;
  }
}

// ---------------------------------------------------------------- varlen segment plan
// seg_base[n] = sum over earlier sequences of max(1, ceil(ceil(len/64)/R)),
// capped at seg_slots, and seg_order = the segment ids sorted by length
// (chunks), longest first, so that workgroups of long segments are dispatched
// before short ones.  A counting sort over min(length, kOrderBuckets - 1); the
// order inside a bucket is arbitrary (segments are independent, so results do
// not depend on it).  Offsets are clamped to [0, T] (seq_extent), so offsets
// that break the documented precondition change outputs but never the bounds
// of any access; the cap keeps every segment id below seg_slots.
constexpr int kOrderBuckets = 1024;

__device__ __forceinline__ int seg_count(int len, int R) {
  const int nc = (len + C - 1) / C;
  return max(1, (nc + R - 1) / R);
}

__global__ __launch_bounds__(1024) void gla_segment_plan(const int32_t *cu, int N, int T, int R, int seg_slots,
                                                         int32_t *seg_base, int32_t *seg_order, int32_t *clear,
                                                         int nclear) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry;
  __shared__ int32_t bucket[kOrderBuckets];
  const int tid = threadIdx.x;
  for (int i = tid; i < nclear; i += 1024) clear[i] = 0;  // the single pass's link table
  if (tid == 0) {
    carry = 0;
    seg_base[0] = 0;
  }
  for (int i = tid; i < kOrderBuckets; i += 1024) bucket[i] = 0;
  __syncthreads();
  // segment table (inclusive block scans of the per-sequence counts)
  for (int base = 0; base < N; base += 1024) {
    const int n = base + tid;
    int cnt = 0;
    if (n < N) {
      int bos, len;
      seq_extent(cu, n, T, bos, len);
      cnt = seg_count(len, R);
    }
    part[tid] = cnt;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int add = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    if (n < N) seg_base[n + 1] = (int32_t)min((long long)carry + part[tid], (long long)seg_slots);
    __syncthreads();
    if (tid == 1023) carry = (int32_t)min((long long)carry + part[1023], (long long)seg_slots);
    __syncthreads();
  }
  // lengths of the segments each sequence actually gets (the walkers cut it the same way)
  for (int n = tid; n < N; n += 1024) {
    int bos, len;
    seq_extent(cu, n, T, bos, len);
    const int nc = (len + C - 1) / C;
    const int cnt = seg_base[n + 1] - seg_base[n];  // written above by this or another thread
    if (cnt <= 0) continue;
    const int sl = (nc + cnt - 1) / cnt;
    for (int s = 0; s < cnt; ++s) atomicAdd(&bucket[min(max(0, min(sl, nc - s * sl)), kOrderBuckets - 1)], 1);
  }
  __syncthreads();
  // start of each length bucket in the order, longest first: an exclusive scan
  // over the buckets from the longest down, one bucket per thread
  static_assert(kOrderBuckets == 1024, "one bucket per thread");
  {
    const int b = kOrderBuckets - 1 - tid;
    const int cnt = bucket[b];
    part[tid] = cnt;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
      const int add = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    bucket[b] = part[tid] - cnt;
  }
  __syncthreads();
  for (int n = tid; n < N; n += 1024) {
    int bos, len;
    seq_extent(cu, n, T, bos, len);
    const int nc = (len + C - 1) / C;
    const int first = seg_base[n];
    const int cnt = seg_base[n + 1] - first;
    if (cnt <= 0) continue;
    const int sl = (nc + cnt - 1) / cnt;
    for (int s = 0; s < cnt; ++s) {
      const int slot = atomicAdd(&bucket[min(max(0, min(sl, nc - s * sl)), kOrderBuckets - 1)], 1);
      seg_order[slot] = first + s;  // slot < seg_base[N] <= seg_slots
    }
  }
}

__global__ __launch_bounds__(256) void gla_clear_words(int32_t *words, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) words[i] = 0;
}

template <bool BF, int KD, bool GH>
hipError_t launch_walk_g(bool local_mode, const WalkParams &p, hipStream_t s) {
  const int NV = (p.V + VT - 1) / VT;
  const int groups = (p.units + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * NV));
  if (local_mode)
    hipLaunchKernelGGL((gla_chunk_local<BF, KD, GH>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((gla_chunk_output<BF, KD, GH>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <bool BF, int KD>
hipError_t launch_walk_t(bool local_mode, const WalkParams &p, hipStream_t s) {
  return p.gate_head ? launch_walk_g<BF, KD, true>(local_mode, p, s) : launch_walk_g<BF, KD, false>(local_mode, p, s);
}

}  // namespace

hipError_t launch_walk_general(bool local_mode, bool bf16, int kd, const WalkParams &p, hipStream_t s) {
  if (p.K > kd || p.vtile != VT) return hipErrorInvalidValue;
  if (bf16) {
    switch (kd) {
      case 32: return launch_walk_t<true, 32>(local_mode, p, s);
      case 64: return launch_walk_t<true, 64>(local_mode, p, s);
      case 128: return launch_walk_t<true, 128>(local_mode, p, s);
    }
  } else {
    switch (kd) {
      case 16: return launch_walk_t<false, 16>(local_mode, p, s);
      case 32: return launch_walk_t<false, 32>(local_mode, p, s);
      case 64: return launch_walk_t<false, 64>(local_mode, p, s);
      case 128: return launch_walk_t<false, 128>(local_mode, p, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_state_scan(const WalkParams &p, hipStream_t s) {
  const int KV4 = p.K * p.V / 4;
  const int per_state = (KV4 + 255) / 256;
  const long long blocks = (long long)p.N * p.HV * per_state;
  if (blocks <= 0 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gla_state_scan, dim3((unsigned)blocks), dim3(256), 0, s, p, per_state);
  return hipGetLastError();
}

hipError_t launch_clear(int32_t *words, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(gla_clear_words, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, s, words, n);
  return hipGetLastError();
}

hipError_t launch_segment_plan(const WalkParams &p, int32_t *seg_base, int32_t *seg_order, hipStream_t s,
                               int32_t *clear, int nclear) {
  hipLaunchKernelGGL(gla_segment_plan, dim3(1), dim3(1024), 0, s, p.cu, p.N, p.T, p.R, p.seg_slots, seg_base,
                     seg_order, clear, nclear);
  return hipGetLastError();
}

}  // namespace gla
