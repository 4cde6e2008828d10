// Host side of the C ABI declared in include/gla.h: validation, workspace
// sizing, the choice of state segments and the launch sequence.
//
// Launch sequence on the caller's stream (page "fla/ops/gla/fused_chunk.py",
// FusedChunkGLAFunction.forward, re-planned for one MI355X):
//   [packed input, several segments possible]  gla_segment_plan
//   [some sequence spans several segments]    gla_chunk_local -> gla_state_scan
//   always                                    gla_chunk_output
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gla.h"
#include "gla_internal.h"

namespace {

using gla::kChunk;
using gla::kVTile;

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev] = cus;
  return cus;
}

bool k_supported(int dtype, int K) {
  if (dtype == GLA_BF16) return K == 32 || K == 64 || K == 128;
  return K == 16 || K == 32 || K == 64 || K == 128;
}

gla_status validate(const gla_problem *p) {
  if (!p) return GLA_ERR_NULL_ARG;
  if (p->B < 0 || p->T < 0 || p->H <= 0 || p->K <= 0 || p->V <= 0 || p->n_seqs < 0) return GLA_ERR_BAD_SHAPE;
  if (p->dtype != GLA_F32 && p->dtype != GLA_BF16) return GLA_ERR_BAD_DTYPE;
  if (!(std::isfinite(p->scale) && p->scale > 0.f)) return GLA_ERR_BAD_SCALE;
  if (p->chunk != kChunk) return GLA_ERR_UNSUPPORTED;
  if (!k_supported(p->dtype, p->K) || p->V % kVTile != 0) return GLA_ERR_UNSUPPORTED;
  if (p->segment_chunks < 0 || (p->packed != 0 && p->packed != 1)) return GLA_ERR_BAD_SHAPE;
  if (p->packed ? p->B != 1 : p->n_seqs != p->B) return GLA_ERR_BAD_SHAPE;
  // element counts must stay addressable
  const double elems = (double)p->B * p->T * p->H * (p->K > p->V ? p->K : p->V);
  if (elems > 9.0e15) return GLA_ERR_BAD_SHAPE;
  return GLA_OK;
}

// How the sequence axis is cut into state segments.
struct Plan {
  bool varlen;
  int N;          // sequences
  int R;          // chunks per segment
  int P;          // segments per sequence (fixed length)
  int seg_slots;  // upper bound on segments over all sequences
  int vtile;      // value columns per workgroup
  bool segmented; // some sequence may span several segments
  size_t ws_state, ws_decay, ws_base, ws_total;
};

Plan make_plan(const gla_problem *p, bool varlen) {
  Plan pl{};
  pl.varlen = varlen;
  pl.N = varlen ? p->n_seqs : p->B;
  const int H = p->H;
  // Value columns per workgroup.  The bf16 walker's 128-column workgroups form
  // the gated operands of a head once for all 128 columns; they are used when
  // they alone fill the device, or when sequences must be cut into segments
  // anyway.  Otherwise 64-column workgroups double the parallelism without
  // segmenting.  GLA_BF16_VTILE=64 / =128 fixes the choice (A/B runs).
  int vtile = kVTile;
  if (gla::bf16_walker_used(p->dtype == GLA_BF16, p->K) && p->V % 128 == 0) {
    const long long rows = (long long)pl.N * H;
    const char *env = getenv("GLA_BF16_VTILE");
    if (env != nullptr && strcmp(env, "64") == 0) vtile = 64;
    else if (env != nullptr && strcmp(env, "128") == 0) vtile = 128;
    else if (varlen || rows * (p->V / 128) >= device_cu_count()) vtile = 128;
    else vtile = rows * (p->V / 64) >= device_cu_count() ? 64 : 128;
  }
  pl.vtile = vtile;
  const int NV = p->V / vtile;
  const long long chunks_total = ((long long)p->T + kChunk - 1) / kChunk;  // varlen: packed axis
  const long long chunks_seq = chunks_total;  // longest possible sequence
  int R = p->segment_chunks;
  if (R == 0) {
    // Enough (segment, head, value slice) workgroups to give every compute
    // unit work; long sequences with few heads are cut into segments.  A
    // 128-column workgroup fills a compute unit on its own.
    const long long target = (vtile == 128 ? 1LL : 2LL) * device_cu_count();
    const long long units_one = (long long)pl.N * H * NV;
    if (!varlen) {
      if (units_one >= device_cu_count() || chunks_seq <= 1) {
        R = (int)(chunks_seq > 0 ? chunks_seq : 1);
      } else {
        long long P = (target + units_one - 1) / units_one;
        if (P > chunks_seq) P = chunks_seq;
        R = (int)((chunks_seq + P - 1) / P);
      }
    } else {
      // packed: about 1.5 segment workgroups per compute unit balances the
      // unequal segment lengths (dispatched longest first) against the extra
      // summary work of cutting more sequences (measured optimum on the
      // 16-sequence U[256, 4096] workload)
      const long long work = (chunks_total + pl.N) * H * NV;  // chunk-slices to spread
      const long long tgt = vtile == 128 ? (3LL * device_cu_count()) / 2 : target;
      long long r = (work + tgt - 1) / tgt;
      if (r < 4) r = 4;
      R = (int)r;
    }
    if (R < 1) R = 1;
  }
  pl.R = R;
  if (!varlen) {
    const long long P = chunks_seq <= 0 ? 1 : (chunks_seq + R - 1) / R;
    pl.P = (int)P;
    pl.seg_slots = pl.N * pl.P;
    pl.segmented = pl.P > 1;
  } else {
    pl.P = 1;
    // every sequence has max(1, ceil(nc/R)) segments; nc <= len/64 + 1
    const long long bound = pl.N + (chunks_total + pl.N + R - 1) / R;
    pl.seg_slots = (int)bound;
    pl.segmented = chunks_total > R;  // a sequence needs more than one segment only if it has > R chunks
  }
  if (pl.segmented) {
    pl.ws_state = (size_t)pl.seg_slots * H * p->K * p->V * sizeof(float);
    pl.ws_decay = (size_t)pl.seg_slots * H * p->K * sizeof(float);
    pl.ws_base = varlen ? (size_t)(pl.N + 1 + pl.seg_slots) * sizeof(int32_t) : 0;  // table + order
  }
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  pl.ws_total = up(pl.ws_state) + up(pl.ws_decay) + up(pl.ws_base);
  return pl;
}

}  // namespace

extern "C" {

const char *gla_status_str(gla_status s) {
  switch (s) {
    case GLA_OK: return "ok";
    case GLA_ERR_NULL_ARG: return "a required pointer is NULL";
    case GLA_ERR_BAD_SHAPE: return "invalid or inconsistent sizes";
    case GLA_ERR_BAD_DTYPE: return "dtype must be GLA_F32 or GLA_BF16";
    case GLA_ERR_BAD_SCALE: return "scale must be finite and > 0";
    case GLA_ERR_UNSUPPORTED: return "unsupported K, V or chunk for the built kernels";
    case GLA_ERR_WORKSPACE: return "workspace missing or too small";
    case GLA_ERR_HIP: return "HIP runtime or launch failure";
  }
  return "unknown status";
}

size_t gla_fwd_workspace_bytes(const gla_problem *p) {
  if (validate(p) != GLA_OK) return (size_t)-1;
  return make_plan(p, p->packed == 1).ws_total;
}

gla_status gla_fwd(const gla_problem *p, const void *q, const void *k, const void *v, const float *g,
                   const float *h0, const int32_t *cu_seqlens, void *o, float *ht, void *workspace,
                   size_t workspace_bytes, void *stream) {
  gla_status st = validate(p);
  if (st != GLA_OK) return st;
  const bool varlen = p->packed == 1;
  if (varlen != (cu_seqlens != nullptr)) return GLA_ERR_NULL_ARG;
  const bool empty_tokens = (long long)p->B * p->T == 0;
  if (!empty_tokens && (!q || !k || !v || !g || !o)) return GLA_ERR_NULL_ARG;
  const int N = varlen ? p->n_seqs : p->B;
  if (N == 0) return GLA_OK;  // nothing to compute and no state to return
  const Plan pl = make_plan(p, varlen);
  if (pl.ws_total > 0 && (workspace == nullptr || workspace_bytes < pl.ws_total)) return GLA_ERR_WORKSPACE;
  if (empty_tokens && ht == nullptr) return GLA_OK;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  gla::WalkParams w{};
  w.q = q; w.k = k; w.v = v; w.g = g; w.h0 = h0; w.cu = cu_seqlens; w.o = o; w.ht = ht;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char *ws = reinterpret_cast<char *>(workspace);
  w.seg_state = pl.segmented ? reinterpret_cast<float *>(ws) : nullptr;
  w.seg_decay = pl.segmented ? reinterpret_cast<float *>(ws + up(pl.ws_state)) : nullptr;
  int32_t *seg_base = (pl.segmented && varlen)
                          ? reinterpret_cast<int32_t *>(ws + up(pl.ws_state) + up(pl.ws_decay))
                          : nullptr;
  w.seg_base = seg_base;
  w.seg_order = seg_base ? seg_base + N + 1 : nullptr;
  w.T = p->T; w.H = p->H; w.K = p->K; w.V = p->V; w.N = N;
  w.R = pl.R;
  w.P = pl.P;
  w.units = (pl.segmented ? pl.seg_slots : (varlen ? N : N * pl.P)) * p->H;
  w.vtile = pl.vtile;
  w.scale = p->scale;
  const bool bf = p->dtype == GLA_BF16;

  if (seg_base && gla::launch_segment_plan(w, seg_base, seg_base + N + 1, s) != hipSuccess) return GLA_ERR_HIP;
  if (pl.segmented) {
    if (gla::launch_walk(true, bf, p->K, w, s) != hipSuccess) return GLA_ERR_HIP;
    if (gla::launch_state_scan(w, s) != hipSuccess) return GLA_ERR_HIP;
  }
  if (gla::launch_walk(false, bf, p->K, w, s) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

}  // extern "C"
