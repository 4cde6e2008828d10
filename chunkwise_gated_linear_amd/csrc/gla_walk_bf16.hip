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
// Layout for gfx950:
//  * The four waves tile the K x 64 state slice as 2 (key halves) x 2 (value
//    halves of 32 columns); wave (kh, nh) keeps S[64kh + ..][32nh + ..] in MFMA
//    accumulators.  Each wave forms a partial output over its key half; the
//    two partials meet in LDS and are summed by the store pass.
//  * qc and kc live in LDS once, token-major (key contiguous).  The key-major
//    operand kc^T of S += kc^T v and the value operand v of A v and kc^T v are
//    read with the LDS transpose read ds_read_b64_tr_b16, so no transposed copy
//    is ever written.
//  * Global traffic uses buffer descriptors per chunk: rows past the end of a
//    sequence read as zero and their output stores are dropped.
//  * The next chunk's q, k, g, v are loaded into registers while the current
//    chunk computes.
#include "gla_device.h"
#include "gla_internal.h"

#include <type_traits>

namespace gla {
namespace {

using namespace dev;

template <int KD, bool OUT>
struct LdsB {
  static constexpr int NQ = KD / 4;                // prologue column quads
  static constexpr int QPW = NQ / 4;               // column quads per wave
  static constexpr int NG = 64 / QPW;              // prologue row groups
  static constexpr int QROW = 2 * KD + 16;         // qc / kc rows (bf16)
  static constexpr int VROW = 2 * VT + 32;         // v rows (bf16): 4 rows x 32 B of one transpose read fall in distinct banks
  static constexpr int OROW = 4 * VT + 16;         // partial outputs (fp32)
  static constexpr int QPL = C * QROW;             // one plane of qc or kc
  static constexpr int OPL = C * OROW;
  static constexpr int oQ = 0;                     // qc hi, lo            (OUT)
  static constexpr int oK = oQ + (OUT ? 2 * QPL : 0);   // kc hi, lo
  static constexpr int oV = oK + 2 * QPL;          // v [token][n]
  static constexpr int oO = oV + C * VROW;         // partial o [kh][i][n] (OUT)
  static constexpr int oDec = oO + (OUT ? 2 * OPL : 0); // a [K]
  static constexpr int BYTES = oDec + 4 * KD;
};

template <bool OUT, int KD>
__device__ __forceinline__ void walk_bf16(const WalkParams &p, char *smem) {
  using L = LdsB<KD, OUT>;
  constexpr int QPW = L::QPW, NG = L::NG, RPG = C / NG;
  constexpr int KH = KD / 2;        // state rows per wave
  constexpr int NKT = KH / 16;      // 16-row k tiles per wave
  constexpr int NKB = KH / 32;      // 32-wide k blocks per wave
  static_assert(KD == 64 || KD == 128, "bf16 walker covers K = 64, 128");
  static_assert(NG * QPW == 64 && RPG * NG == C, "prologue mapping");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lg = lane >> 4;
  const int kh = wave >> 1, nh = wave & 1;

  // ---- (segment, head, value slice) of this workgroup; value slices of one
  // unit are 8 workgroup ids apart so they run on the same XCD and share L2.
  const int NV = p.V / VT;
  const int b = blockIdx.x;
  const int grp = b / (8 * NV), rem = b - grp * (8 * NV);
  const int vt = rem >> 3;
  const int unit = grp * 8 + (rem & 7);
  if (unit >= p.units) return;
  const int seg = unit / p.H, h = unit - seg * p.H;
  SegInfo si;
  if (!locate(p, seg, si)) return;
  if (!OUT && si.s >= si.nseg - 1) return;
  const int nchunks = (si.len + C - 1) / C;
  const int c_begin = si.s * p.R;
  const int c_end = min(c_begin + p.R, nchunks);
  const int H = p.H, V = p.V;
  const int v0 = vt * VT;
  const int64_t rowK = (int64_t)H * KD, rowV = (int64_t)H * V;

  // ---- state block of this lane: S[KH kh + 16kt + 4lg + r][v0 + 32nh + 16nt + l16]
  f32x4_t S[NKT][2];
  {
    const float *src = nullptr;
    if (OUT) {
      if (si.s == 0) {
        if (p.h0) src = p.h0 + ((int64_t)si.n * H + h) * KD * V;
      } else {
        src = p.seg_state + ((int64_t)(si.first + si.s - 1) * H + h) * KD * V;
      }
    }
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          S[kt][nt][r] = src ? src[(int64_t)(KH * kh + 16 * kt + 4 * lg + r) * V + v0 + 32 * nh + 16 * nt + l16] : 0.f;
  }

  // ---- prologue mapping: wave w gates key columns [32w, 32w+32) (K=128) of all 64
  // rows; lane = rg * QPW + quad: rows rg*RPG .. +RPG-1, columns 4cq .. 4cq+3.
  // The running products across row groups stay inside the wave (lane shuffles).
  // v: row tid/4, 16 columns.
  const int cq = wave * QPW + lane % QPW, rg = lane / QPW;
  const int voff_g = (int)((rg * RPG * rowK + 4 * cq) * 4);
  const int voff_k = (int)((rg * RPG * rowK + 4 * cq) * 2);
  const int vrow = tid >> 2, vcol = 16 * (tid & 3);
  const int voff_v = (int)((vrow * rowV + vcol) * 2);
  const int step_g = (int)(rowK * 4), step_k = (int)(rowK * 2);
  const int colq = kperm_bf(4 * cq) * 2;

  // Software pipeline over chunks: while chunk c runs on the matrix cores, the
  // gated operands of chunk c+1 are formed in registers and the raw inputs of
  // chunk c+2 are loaded.  Loads past the sequence (or past the segment) read
  // zeros, so the pipeline runs the same instruction stream every iteration.
  u32x4_t rgG[RPG];                       // raw inputs of the chunk to gate next
  u32x2_t rgQ[RPG], rgK[RPG];
  u32x4_t rgV[2];
  u32x2_t gQh[RPG], gQl[RPG], gKh[RPG], gKl[RPG];   // gated operands of the chunk to compute next
  u32x4_t gV[2];
  f32x4_t gDec = {1.f, 1.f, 1.f, 1.f};

  float seg_decay[4] = {1.f, 1.f, 1.f, 1.f};
  const float scale = p.scale;

  // gate: decays of the chunk and the gated, split q and k in registers.  It
  // runs in stages so that its vector work can be spread between the matrix
  // instructions of the previous chunk.
  float gE[RPG][4], gPl[RPG][4], gRl[RPG][4], gSuf[4], gFq[4];
  auto gate_a = [&]() {  // exp(g) and running products inside the row group
#pragma unroll
    for (int r = 0; r < RPG; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) gE[r][j] = __expf(__uint_as_float(rgG[r][j]));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      gPl[0][j] = gE[0][j];
#pragma unroll
      for (int r = 1; r < RPG; ++r) gPl[r][j] = gPl[r - 1][j] * gE[r][j];
      gRl[RPG - 1][j] = 1.f;
#pragma unroll
      for (int r = RPG - 2; r >= 0; --r) gRl[r][j] = gRl[r + 1][j] * gE[r + 1][j];
    }
  };
  auto gate_b = [&]() {  // products over row groups: inclusive scan across the lanes of a column quad
    float incl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) incl[j] = gPl[RPG - 1][j];
#pragma unroll
    for (int d = 1; d < NG; d *= 2) {
      const int src = (lane - d * QPW) < 0 ? lane : lane - d * QPW;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float y = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src, __float_as_int(incl[j])));
        incl[j] *= (rg >= d) ? y : 1.f;
      }
    }
    const int src_pre = rg > 0 ? lane - QPW : lane;
    const int src_tot = (NG - 1) * QPW + lane % QPW;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float y = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src_pre, __float_as_int(incl[j])));
      const float pre = rg > 0 ? y : 1.f;
      const float tot = __int_as_float(__builtin_amdgcn_ds_bpermute(4 * src_tot, __float_as_int(incl[j])));
      gSuf[j] = tot * __builtin_amdgcn_rcpf(incl[j]);
      gFq[j] = OUT ? scale * pre * __builtin_amdgcn_rcpf(tot) : 0.f;
      gDec[j] = tot;
    }
    if (!OUT && rg == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) seg_decay[j] *= gDec[j];
    }
  };
  auto gate_rows = [&](int r0, int r1) {  // gated, split q and k of rows [r0, r1)
#pragma unroll
    for (int r = r0; r < r1; ++r) {
      float kc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float kk = (j & 1) ? bf_hi(rgK[r][j >> 1]) : bf_lo(rgK[r][j >> 1]);
        kc[j] = kk * (gRl[r][j] * gSuf[j]);
      }
      split4(kc, gKh[r], gKl[r]);
      if (OUT) {
        float qc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float qq = (j & 1) ? bf_hi(rgQ[r][j >> 1]) : bf_lo(rgQ[r][j >> 1]);
          qc[j] = qq * (gPl[r][j] * gFq[j]);
        }
        split4(qc, gQh[r], gQl[r]);
      }
    }
  };
  auto gate = [&]() {
    gate_a();
    gate_b();
    gate_rows(0, RPG);
    gV[0] = rgV[0];
    gV[1] = rgV[1];
  };
  // loads of one chunk in four parts (g first half, g second half, k and q, v)
  auto load_part = [&](int c, int part) {
    const int64_t t0 = (int64_t)si.bos + (int64_t)c * C;
    const int64_t valid = c < c_end ? min(C, si.len - c * C) : 0;
    const int64_t headK = (int64_t)h * KD, headV = (int64_t)h * V + v0;
    if (part == 0 || part == 1) {
      const __amdgpu_buffer_rsrc_t rG = make_rsrc(p.g + t0 * rowK + headK, (valid * rowK - headK) * 4);
#pragma unroll
      for (int r = part * RPG / 2; r < (part + 1) * RPG / 2; ++r) rgG[r] = buf_ld128(rG, voff_g + r * step_g);
    } else if (part == 2) {
      const __amdgpu_buffer_rsrc_t rK = make_rsrc((const uint16_t *)p.k + t0 * rowK + headK, (valid * rowK - headK) * 2);
#pragma unroll
      for (int r = 0; r < RPG; ++r) rgK[r] = buf_ld64(rK, voff_k + r * step_k);
      if (OUT) {
        const __amdgpu_buffer_rsrc_t rQ = make_rsrc((const uint16_t *)p.q + t0 * rowK + headK, (valid * rowK - headK) * 2);
#pragma unroll
        for (int r = 0; r < RPG; ++r) rgQ[r] = buf_ld64(rQ, voff_k + r * step_k);
      }
    } else {
      const __amdgpu_buffer_rsrc_t rV = make_rsrc((const uint16_t *)p.v + t0 * rowV + headV, (valid * rowV - headV) * 2);
      rgV[0] = buf_ld128(rV, voff_v);
      rgV[1] = buf_ld128(rV, voff_v + 16);
    }
  };

  auto write_gated = [&]() {
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
      const int off = (rg * RPG + r) * L::QROW + colq;
      lds_st<u32x2_t>(smem + L::oK, off, gKh[r]);
      lds_st<u32x2_t>(smem + L::oK + L::QPL, off, gKl[r]);
      if (OUT) {
        lds_st<u32x2_t>(smem + L::oQ, off, gQh[r]);
        lds_st<u32x2_t>(smem + L::oQ + L::QPL, off, gQl[r]);
      }
    }
    lds_st<u32x4_t>(smem + L::oV, vrow * L::VROW + vcol * 2, gV[0]);
    lds_st<u32x4_t>(smem + L::oV, vrow * L::VROW + vcol * 2 + 16, gV[1]);
    if (rg == 0) lds_st<f32x4_t>(smem + L::oDec, 16 * cq, gDec);
  };

  // lane bases of the matrix-phase LDS accesses
  // The token (contraction) index of A v and kc^T v is taken in the order of
  // the score accumulators: within a 32-token block jb, lane group lg holds
  // tokens 32jb + 16h + 4lg + e (h = 0, 1; e = 0..3) -- so the score tiles
  // feed A v straight from registers.  Transpose reads deliver that order.
  const int base_q = l16 * L::QROW + 16 * lg;                                  // normal reads, rows of qc / kc
  const int base_vt = (4 * lg + (l16 >> 2)) * L::VROW + (32 * nh + 4 * (l16 & 3)) * 2;   // transpose reads of v
  const int base_kt = (4 * lg + (l16 >> 2)) * L::QROW + (KH * kh + 8 * (l16 & 3)) * 2;   // transpose reads of kc
  const int base_o = 4 * lg * L::OROW + (32 * nh + l16) * 4 + kh * L::OPL;     // partial o writes
  const int base_d = (KH * kh + 4 * lg) * 4;                                   // decay reads

  // ---- pipeline fill
  if (c_begin < c_end) {
    for (int part = 0; part < 4; ++part) load_part(c_begin, part);
    gate();
    for (int part = 0; part < 4; ++part) load_part(c_begin + 1, part);
  }

  for (int c = c_begin; c < c_end; ++c) {
    write_gated();
    __syncthreads();  // chunk c operands visible

    // ---- S' = diag(a) S
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      const f32x4_t a4 = lds_ld<f32x4_t>(smem + L::oDec, base_d + 64 * kt);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[kt][nt][r] *= a4[r];
    }
    // ---- v fragments (B operand of A v and kc^T v)
    u32x4_t vf[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int off = base_vt + 32 * jb * L::VROW + 32 * nt;
        const u32x2_t x0 = lds_tr16(smem + L::oV + off);
        const u32x2_t x1 = lds_tr16(smem + L::oV + off + 16 * L::VROW);
        vf[nt][jb] = u32x4_t{x0[0], x0[1], x1[0], x1[1]};
      }

    f32x4_t o[4][2];
    if constexpr (OUT) {
      // ---- this wave's key half: scores A_kh^T = kc qc^T (lower tiles) and o += qc S'
      f32x4_t A[10];  // tile (it, jt), jt <= it, at index it*(it+1)/2 + jt
#pragma unroll
      for (int t = 0; t < 10; ++t) A[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) o[it][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int col = 64 * (NKB * kh + kb);
        u32x4_t qh[4], ql[4], kh4[4], kl4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int off = base_q + 16 * t * L::QROW + col;
          qh[t] = lds_ld<u32x4_t>(smem + L::oQ, off);
          ql[t] = lds_ld<u32x4_t>(smem + L::oQ + L::QPL, off);
          kh4[t] = lds_ld<u32x4_t>(smem + L::oK, off);
          kl4[t] = lds_ld<u32x4_t>(smem + L::oK + L::QPL, off);
        }
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
          for (int jt = 0; jt <= it; ++jt) {
            f32x4_t &acc = A[it * (it + 1) / 2 + jt];
            acc = mfma_bf(kl4[jt], qh[it], acc);
            acc = mfma_bf(kh4[jt], ql[it], acc);
            acc = mfma_bf(kh4[jt], qh[it], acc);
          }
        u32x4_t sh[2], sl[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const float s8[8] = {S[2 * kb][nt][0], S[2 * kb][nt][1], S[2 * kb][nt][2], S[2 * kb][nt][3],
                               S[2 * kb + 1][nt][0], S[2 * kb + 1][nt][1], S[2 * kb + 1][nt][2], S[2 * kb + 1][nt][3]};
          u32x2_t h0, l0, h1, l1;
          split4(s8, h0, l0);
          split4(s8 + 4, h1, l1);
          sh[nt] = u32x4_t{h0[0], h0[1], h1[0], h1[1]};
          sl[nt] = u32x4_t{l0[0], l0[1], l1[0], l1[1]};
        }
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            o[it][nt] = mfma_bf(ql[it], sh[nt], o[it][nt]);
            o[it][nt] = mfma_bf(qh[it], sl[nt], o[it][nt]);
            o[it][nt] = mfma_bf(qh[it], sh[nt], o[it][nt]);
          }
        // next chunk's gating, spread over the matrix work of this one
        if (kb == 0) gate_a();
        if (kb == NKB - 1) gate_b();
        __builtin_amdgcn_sched_barrier(0);
        if (kb == 0) {
          load_part(c + 2, 0);
          load_part(c + 2, 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ---- o += A_kh v: causal mask, split, scores straight from the accumulators
      // (lane: query i = 16it + l16, keys j = 16jt + 4lg + r)
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int jb = 0; jb <= it / 2; ++jb) {
          float a8[8];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int jt = 2 * jb + hh;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              float x = 0.f;
              if (jt < it) x = A[it * (it + 1) / 2 + jt][r];
              else if (jt == it) x = (4 * lg + r <= l16) ? A[it * (it + 1) / 2 + jt][r] : 0.f;
              a8[4 * hh + r] = x;
            }
          }
          u32x2_t h0, l0, h1, l1;
          split4(a8, h0, l0);
          split4(a8 + 4, h1, l1);
          const u32x4_t ah = {h0[0], h0[1], h1[0], h1[1]};
          const u32x4_t al = {l0[0], l0[1], l1[0], l1[1]};
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            o[it][nt] = mfma_bf(al, vf[nt][jb], o[it][nt]);
            o[it][nt] = mfma_bf(ah, vf[nt][jb], o[it][nt]);
          }
        }
      gate_rows(0, RPG / 2);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      gate_a();
      gate_b();
      __builtin_amdgcn_sched_barrier(0);
      load_part(c + 2, 0);
      load_part(c + 2, 1);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- S = S' + kc^T v   (kc^T rows via transpose reads of the token-major kc)
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const int off = base_kt + 32 * jb * L::QROW + (32 * (kt >> 1) + 4 * (kt & 1)) * 2;
        const u32x2_t h0 = lds_tr16(smem + L::oK + off);
        const u32x2_t h1 = lds_tr16(smem + L::oK + off + 16 * L::QROW);
        const u32x2_t g0 = lds_tr16(smem + L::oK + L::QPL + off);
        const u32x2_t g1 = lds_tr16(smem + L::oK + L::QPL + off + 16 * L::QROW);
        const u32x4_t ah = {h0[0], h0[1], h1[0], h1[1]};
        const u32x4_t al = {g0[0], g0[1], g1[0], g1[1]};
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          S[kt][nt] = mfma_bf(al, vf[nt][jb], S[kt][nt]);
          S[kt][nt] = mfma_bf(ah, vf[nt][jb], S[kt][nt]);
        }
      }
    }
    gate_rows(OUT ? RPG / 2 : 0, RPG);
    gV[0] = rgV[0];
    gV[1] = rgV[1];
    __builtin_amdgcn_sched_barrier(0);
    load_part(c + 2, 2);
    load_part(c + 2, 3);
    __builtin_amdgcn_sched_barrier(0);

    if constexpr (OUT) {
      // ---- partial o -> LDS [kh][i][n] (fp32)
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            lds_st<float>(smem + L::oO, base_o + (16 * it + r) * L::OROW + 64 * nt, o[it][nt][r]);
    }
    __syncthreads();  // partial outputs visible; every read of chunk c's operands is done

    if constexpr (OUT) {
      // ---- sum the two key-half partials, round to bf16, store 32 B per thread
      const int64_t t0 = (int64_t)si.bos + (int64_t)c * C;
      const int64_t valid = min(C, si.len - c * C);
      const int64_t headV = (int64_t)h * V + v0;
      const __amdgpu_buffer_rsrc_t rO = make_rsrc((uint16_t *)p.o + t0 * rowV + headV, (valid * rowV - headV) * 2);
      const int orow = tid >> 2, ocol = 16 * (tid & 3);
      uint32_t w[8];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const f32x4_t a0 = lds_ld<f32x4_t>(smem + L::oO, orow * L::OROW + (ocol + 4 * x) * 4);
        const f32x4_t a1 = lds_ld<f32x4_t>(smem + L::oO + L::OPL, orow * L::OROW + (ocol + 4 * x) * 4);
        w[2 * x] = pack_bf16(a0[0] + a1[0], a0[1] + a1[1]);
        w[2 * x + 1] = pack_bf16(a0[2] + a1[2], a0[3] + a1[3]);
      }
      const int so = (int)((orow * rowV + ocol) * 2);
      buf_st128(rO, so, u32x4_t{w[0], w[1], w[2], w[3]});
      buf_st128(rO, so + 16, u32x4_t{w[4], w[5], w[6], w[7]});
    }
  }

  // ================= results of the segment
  float *dst = nullptr;
  if (OUT) {
    if (p.ht != nullptr && si.s == si.nseg - 1) dst = p.ht + ((int64_t)si.n * H + h) * KD * V;
  } else {
    const int slot = si.first + si.s;
    dst = p.seg_state + ((int64_t)slot * H + h) * KD * V;
    if (vt == 0 && rg == 0)
      *reinterpret_cast<f32x4_t *>(p.seg_decay + ((int64_t)slot * H + h) * KD + 4 * cq) =
          f32x4_t{seg_decay[0], seg_decay[1], seg_decay[2], seg_decay[3]};
  }
  if (dst) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dst[(int64_t)(KH * kh + 16 * kt + 4 * lg + r) * V + v0 + 32 * nh + 16 * nt + l16] = S[kt][nt][r];
  }
}

template <int KD>
__global__ __launch_bounds__(kThreads, 1) void gla_chunk_output_bf16(WalkParams p) {
  __shared__ __attribute__((aligned(16))) char smem[LdsB<KD, true>::BYTES];
  walk_bf16<true, KD>(p, smem);
}

template <int KD>
__global__ __launch_bounds__(kThreads, 1) void gla_chunk_local_bf16(WalkParams p) {
  __shared__ __attribute__((aligned(16))) char smem[LdsB<KD, false>::BYTES];
  walk_bf16<false, KD>(p, smem);
}

template <int KD>
hipError_t launch_t(bool local_mode, const WalkParams &p, hipStream_t s) {
  const int NV = p.V / VT;
  const int groups = (p.units + 7) / 8;
  const dim3 grid((unsigned)(groups * 8 * NV));
  if (local_mode)
    hipLaunchKernelGGL(gla_chunk_local_bf16<KD>, grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(gla_chunk_output_bf16<KD>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool walk_bf16_supported(int K) { return K == 64 || K == 128; }

hipError_t launch_walk_bf16(bool local_mode, int K, const WalkParams &p, hipStream_t s) {
  if (K == 128) return launch_t<128>(local_mode, p, s);
  if (K == 64) return launch_t<64>(local_mode, p, s);
  return hipErrorInvalidValue;
}

}  // namespace gla
