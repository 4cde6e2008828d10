// Device helpers shared by the kernels (gla_kernels.hip, gla_walk_bf16.hip, gla_bwd.hip, gla_wy.hip).
#pragma once

#include "gla_internal.h"

namespace gla {
namespace dev {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int C = kChunk;
constexpr int VT = kVTile;

// ---------------------------------------------------------------- helpers
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest-even) and pack them, x0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float x0, float x1) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t h;
  h[0] = (__bf16)x0;
  h[1] = (__bf16)x1;
  return __builtin_bit_cast(uint32_t, h);
}

// x rounded to bf16 (nearest-even), as a float: the conversion writes the bf16
// into the upper half of the word over a zero lower half, which is that float.
// (Written out because the compiler otherwise forms it from the packed pair as
// a second conversion plus a shift.)  The compiler does not insert wait states
// before inline asm, so x must come from ordinary VALU arithmetic, never
// straight from an MFMA result or a transcendental.
__device__ __forceinline__ float bf16_round_valu(float x) {
  float r;
  asm("v_cvt_pk_bf16_f32 %0, 0, %1" : "=v"(r) : "v"(x));
  return r;
}

// x - (one bf16 half of the packed word w), from the word itself: a bf16 dot
// product of w with (-1, 0) or (0, -1), accumulated onto x.  The product is
// exact and so is the difference (the remainder of rounding x to bf16 is a
// float), so this equals x - bf_lo(w) / x - bf_hi(w) in one instruction.
// The pair (-1, 0) is the word 0x0000bf80, which the compiler encodes as the
// inline constant -1.0; the hardware reads that operand as the float -1.0,
// i.e. the word 0xbf800000 = (0, -1).  The word is therefore kept in a scalar
// register the compiler cannot see into.
__device__ __forceinline__ float minus_bf_lo(uint32_t w, float x) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  uint32_t m = 0x0000bf80u;
  asm("" : "+s"(m));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, m), x, false);
}
__device__ __forceinline__ float minus_bf_hi(uint32_t w, float x) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, 0xbf800000u),
                                         x, false);
}

// Split 4 floats into bf16 hi (nearest) and bf16 lo (nearest of the remainder).
// The dot instruction accumulates into its destination, so this form suits
// values that die at the split; a value that stays live (the carried state)
// would first be copied, and split4_sub / split4_valu are used for it.
__device__ __forceinline__ void split4(const float x[4], u32x2_t &hi, u32x2_t &lo) {
  hi[0] = pack_bf16(x[0], x[1]);
  hi[1] = pack_bf16(x[2], x[3]);
  lo[0] = pack_bf16(minus_bf_lo(hi[0], x[0]), minus_bf_hi(hi[0], x[1]));
  lo[1] = pack_bf16(minus_bf_lo(hi[1], x[2]), minus_bf_hi(hi[1], x[3]));
}
// The same split with the remainders formed by subtraction.
__device__ __forceinline__ void split4_sub(const float x[4], u32x2_t &hi, u32x2_t &lo) {
  hi[0] = pack_bf16(x[0], x[1]);
  hi[1] = pack_bf16(x[2], x[3]);
  lo[0] = pack_bf16(x[0] - bf_lo(hi[0]), x[1] - bf_hi(hi[0]));
  lo[1] = pack_bf16(x[2] - bf_lo(hi[1]), x[3] - bf_hi(hi[1]));
}
// The subtraction split for x computed by ordinary VALU arithmetic (see
// bf16_round_valu): one instruction fewer per pair than split4_sub.
__device__ __forceinline__ void split4_valu(const float x[4], u32x2_t &hi, u32x2_t &lo) {
  hi[0] = pack_bf16(x[0], x[1]);
  hi[1] = pack_bf16(x[2], x[3]);
  lo[0] = pack_bf16(x[0] - bf16_round_valu(x[0]), x[1] - bf_hi(hi[0]));
  lo[1] = pack_bf16(x[2] - bf16_round_valu(x[2]), x[3] - bf_hi(hi[1]));
}

__device__ __forceinline__ f32x4_t mfma_bf(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// An int the compiler cannot see through: keeps a per-lane base offset in a
// register instead of letting it be folded with constants into each access.
__device__ __forceinline__ int opaque_int(int x) {
  asm("" : "+v"(x));
  return x;
}

template <typename T>
__device__ __forceinline__ T lds_ld(const char *base, int byte_off) {
  return *reinterpret_cast<const T *>(base + byte_off);
}
template <typename T>
__device__ __forceinline__ void lds_st(char *base, int byte_off, T v) {
  *reinterpret_cast<T *>(base + byte_off) = v;
}

// Storage column of contraction index p along K (bf16 layout).  Within each
// 32-block, p = 16h + 4G + r is stored at 8G + 4h + r so that the eight
// elements lane group G feeds to one 16x16x32 MFMA are contiguous; the
// element order matches the accumulator layout of the state (rows 4G + r of
// k-tiles 2b and 2b+1), which is what lets the state registers act directly
// as the B operand of qc S'.
__device__ __forceinline__ int kperm_bf(int p) {
  return (p & ~31) | (((p >> 2) & 3) << 3) | (((p >> 4) & 1) << 2) | (p & 3);
}

// ---------------------------------------------------------------- locate a segment
// Token range of packed sequence n, clamped to [0, T]: offsets that break the
// documented precondition (non-decreasing, cu[N] = T) give wrong outputs but
// never an access outside the caller's buffers.
__device__ __forceinline__ void seq_extent(const int32_t *cu, int n, int T, int &bos, int &len) {
  const int a = min(max(cu[n], 0), T);
  const int b = min(max(cu[n + 1], a), T);
  bos = a;
  len = b - a;
}

struct SegInfo {
  int n, s, nseg, first, len;
  int64_t bos;  // first token of the sequence on the flattened [B*T] token axis
};

__device__ __forceinline__ bool locate(const WalkParams &p, int seg, SegInfo &si) {
  if (p.seg_base == nullptr) {
    si.n = seg / p.P;
    si.s = seg - si.n * p.P;
    if (si.n >= p.N) return false;
    si.nseg = p.P;
    si.first = si.n * p.P;
  } else {
    const int total = p.seg_base[p.N];  // <= seg_slots (the segment plan caps it)
    if (seg >= total) return false;
    if (p.seg_order != nullptr) seg = p.seg_order[seg];  // longest segments are dispatched first
    int lo = 0, hi = p.N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.seg_base[mid] <= seg) lo = mid; else hi = mid - 1;
    }
    si.n = lo;
    si.first = p.seg_base[lo];
    si.nseg = p.seg_base[lo + 1] - si.first;
    si.s = seg - si.first;
    if (si.s < 0 || si.s >= si.nseg) return false;
  }
  if (p.cu != nullptr) {
    int bos, len;
    seq_extent(p.cu, si.n, p.T, bos, len);
    si.bos = bos;
    si.len = len;
  } else {
    si.bos = (int64_t)si.n * p.T;
    si.len = p.T;
  }
  // every lane of the workgroup holds the same values; say so, so that they
  // live in scalar registers (buffer descriptors built from them must be uniform)
  si.n = __builtin_amdgcn_readfirstlane(si.n);
  si.s = __builtin_amdgcn_readfirstlane(si.s);
  si.nseg = __builtin_amdgcn_readfirstlane(si.nseg);
  si.first = __builtin_amdgcn_readfirstlane(si.first);
  si.len = __builtin_amdgcn_readfirstlane(si.len);
  const uint32_t blo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)si.bos);
  const uint32_t bhi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)si.bos >> 32));
  si.bos = (int64_t)(((uint64_t)bhi << 32) | blo);
  return true;
}


// ---------------------------------------------------------------- buffer access
// Raw buffer descriptor over `bytes` bytes from `base` (word 3 as for the gfx9
// family).  Loads past `bytes` return zero and stores past it are dropped,
// which is how partial chunks are padded / clipped without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
  n = __builtin_amdgcn_readfirstlane(n);
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t au = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(a >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(au), (short)0, n, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_ld128(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2_t buf_ld64(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ void buf_st128(__amdgpu_buffer_rsrc_t r, int off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, off, 0, 0);
}
// Nontemporal store (cache policy NT): for output written once and not read back.
__device__ __forceinline__ void buf_st128_nt(__amdgpu_buffer_rsrc_t r, int off, u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, off, 0, 2);
}
// fp32 quads with cache policy AUX: 0 plain; 16 (sc1) device scope, the form
// a relaxed agent-scope atomic load or store takes on this GPU (no compute
// unit or die serves it from a private copy)
template <int AUX>
__device__ __forceinline__ f32x4_t buf_ldf4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ void buf_stf4(__amdgpu_buffer_rsrc_t r, int off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v),
                                         r, off, 0, AUX);
}
constexpr int kDeviceScope = 16;
__device__ __forceinline__ void buf_st64(__amdgpu_buffer_rsrc_t r, int off, u32x2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)), v), r, off, 0, 0);
}

// ---------------------------------------------------------------- exact segment re-evaluation
// Four consecutive elements (bf16 or fp32 storage) as floats.
template <bool BF>
__device__ __forceinline__ f32x4_t load4(const void *base, int64_t idx) {
  if constexpr (BF) {
    const u32x2_t w = *reinterpret_cast<const u32x2_t *>(reinterpret_cast<const uint16_t *>(base) + idx);
    return f32x4_t{bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1])};
  } else {
    return *reinterpret_cast<const f32x4_t *>(reinterpret_cast<const float *>(base) + idx);
  }
}
template <bool BF>
__device__ __forceinline__ float load1(const void *base, int64_t idx) {
  if constexpr (BF) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(base)[idx] << 16);
  else return reinterpret_cast<const float *>(base)[idx];
}

// Token-by-token re-evaluation of one (segment, head, value slice): the
// recurrence itself, S = diag(exp(g_t)) S + k_t v_t^T and o_t = scale q_t^T S.
// The walkers run it after their chunk loop for a segment in which some key
// decayed by more than kMinChunkDecay over one chunk, beyond the fp32 range of
// the factorised in-chunk form.
//   OUT:  from the segment's start state (h0, or the start state the scan left
//         in seg_state), rewrites o (or the key block's partial) for every token
//         of the segment.
//   !OUT: from a zero state, forms the segment summary, and writes the per-key
//         product of decays (value slice 0).
// With `stage` (the caller's [KD][VW] fp32 staging area) the final state is
// written there, for the caller to store as ht or as the summary.
// Wave w < VW / 16 takes columns v0 + 16 w + lane % 16; the four lane groups
// lane / 16 hold contiguous quarters of the KD keys and are summed by shuffles.
template <int KD, bool BF, bool OUT>
__device__ void exact_segment(const WalkParams &p, const SegInfo &si, int h, int v0, int VW, int c_begin,
                              int c_end, int wave, int vt, float *stage) {
  if (wave >= VW / 16) return;
  constexpr int KQ = KD / 4;  // keys per lane group
  const int lane = threadIdx.x & 63, l16 = lane & 15, kg = lane >> 4;
  const int col = v0 + 16 * wave + l16;
  const bool col_ok = col < p.V;
  const int nkeys = p.K;
  // h is the value head; q, k are read from key head h / G
  const int64_t rowK = (int64_t)p.H * p.Kmem, rowV = (int64_t)p.HV * p.V;
  const int64_t headK = (int64_t)(h / p.G) * p.Kmem + p.koff, headV = (int64_t)h * p.V + col;
  const int64_t rowG = p.gate_head ? (int64_t)p.HV : (int64_t)p.HV * p.Kmem;
  const int64_t headG = p.gate_head ? (int64_t)h : (int64_t)h * p.Kmem + p.koff;
  const float *src = nullptr;
  if (OUT) {
    if (si.s == 0) {
      if (p.h0) src = p.h0 + (((int64_t)si.n * p.HV + h) * p.Kmem + p.koff) * p.V;
    } else {
      src = p.seg_state + ((int64_t)(si.first + si.s - 1) * p.HV + h) * nkeys * p.V;
    }
  }
  float st[KQ], dec[KQ];
#pragma unroll
  for (int j = 0; j < KQ; ++j) {
    const int key = kg * KQ + j;
    st[j] = (src != nullptr && col_ok && key < nkeys) ? src[(int64_t)key * p.V + col] : 0.f;
    dec[j] = 1.f;
  }
  const int t_end = min(c_end * C, si.len);
  for (int t = c_begin * C; t < t_end; ++t) {
    const int64_t tok = si.bos + t;
    const float vv = col_ok ? load1<BF>(p.v, tok * rowV + headV) : 0.f;
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < KQ; j += 4) {
      const int key = kg * KQ + j;  // a quad of keys is all real or all padding
      if (key < nkeys) {
        const int64_t kidx = tok * rowK + headK + key;
        f32x4_t g4;
        if (p.gate_head) {
          const float x = p.g[tok * rowG + headG];
          g4 = f32x4_t{x, x, x, x};
        } else {
          g4 = *reinterpret_cast<const f32x4_t *>(p.g + tok * rowG + headG + key);
        }
        const f32x4_t k4 = load4<BF>(p.k, kidx);
        f32x4_t q4 = {0.f, 0.f, 0.f, 0.f};
        if (OUT) q4 = load4<BF>(p.q, kidx);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float e = __expf(g4[r]);
          st[j + r] = e * st[j + r] + k4[r] * vv;
          if (OUT) part += q4[r] * st[j + r];
          else dec[j + r] *= e;
        }
      }
    }
    if constexpr (OUT) {
      part += __shfl_xor(part, 16);  // sum over the four key quarters
      part += __shfl_xor(part, 32);
      if (kg == 0 && col_ok) {
        float ov = p.scale * part;
        const int64_t oidx = tok * rowV + headV;
        if (p.o_part != nullptr) {
          p.o_part[oidx] = ov;
        } else {
          if (p.o_add != nullptr) ov += p.o_add[oidx];
          if constexpr (BF) reinterpret_cast<__bf16 *>(p.o)[oidx] = (__bf16)ov;
          else reinterpret_cast<float *>(p.o)[oidx] = ov;
        }
      }
    }
  }
  if (!OUT && vt == 0 && wave == 0 && l16 == 0) {
    float *dd = p.seg_decay + ((int64_t)(si.first + si.s) * p.HV + h) * nkeys;
#pragma unroll
    for (int j = 0; j < KQ; ++j)
      if (kg * KQ + j < nkeys) dd[kg * KQ + j] = dec[j];
  }
  if (stage != nullptr) {
#pragma unroll
    for (int j = 0; j < KQ; ++j) stage[(kg * KQ + j) * VW + 16 * wave + l16] = st[j];
  }
}

// LDS transposing read of four 16-bit elements (ds_read_b64_tr_b16).  Within
// each group of 16 lanes, lane j receives component j%4 of the 8-byte words
// addressed by lanes j/4, j/4+4, j/4+8 and j/4+12 of its group.
__device__ __forceinline__ u32x2_t lds_tr16(const char *p) {
  typedef short v4i16_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
  const lds_v4i16_t *lp = (const lds_v4i16_t *)(const __attribute__((address_space(3))) char *)p;
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_v4i16_t *>(lp)));
}

// ---------------------------------------------------------------- coherence
// Sets bits in the caller-visible status word (a vector-memory atomic OR from
// one lane; the word is only ever OR-ed, never cleared, by the kernels).
__device__ __forceinline__ void report_status(uint32_t *status, uint32_t bits, int lane) {
  if (lane == 0) __hip_atomic_fetch_or(status, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Device-coherent accesses for data that one workgroup publishes to another
// within a launch: agent-scope atomic loads and stores, which no compute unit
// or die keeps a private cached copy of (plain accesses would rely on cache
// write-back and invalidation reaching every line of the other die's L2).
__device__ __forceinline__ float ld_agent(const float *p) {
  return __uint_as_float(
      __hip_atomic_load(reinterpret_cast<const uint32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ f32x4_t ld_agent4(const float *p) {
  const uint64_t *q = reinterpret_cast<const uint64_t *>(p);
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x4_t{__uint_as_float((uint32_t)a), __uint_as_float((uint32_t)(a >> 32)), __uint_as_float((uint32_t)b),
                 __uint_as_float((uint32_t)(b >> 32))};
}
__device__ __forceinline__ void st_agent4(float *p, const f32x4_t &v) {
  uint64_t *q = reinterpret_cast<uint64_t *>(p);
  const uint64_t a = (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32);
  const uint64_t b = (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32);
  __hip_atomic_store(q, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dev
}  // namespace gla
