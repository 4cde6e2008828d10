// Host side of the C ABI declared in include/gla.h: validation, workspace
// sizing, the choice of state segments and key blocks, and the launch sequence.
//
// Launch sequence on the caller's stream (page "fla/ops/gla/fused_chunk.py",
// FusedChunkGLAFunction.forward, re-planned for one MI355X):
//   [packed input, several segments possible]  gla_segment_plan
//   per key block (one, or two when K > 128):
//     [some sequence spans several segments]   gla_chunk_local -> gla_state_scan
//     always                                   gla_chunk_output
//
// Backward (page "fla/ops/gla/fused_chunk.py", FusedChunkGLAFunction.backward):
//   [packed input]                       gla_segment_plan (one chunk per segment)
//   [packed input, chained scan]         gla_bwd_chain_plan: chains ordered by length
//   per key block (K > 128: two) and value slice (V > 128: 128 columns each):
//     [chained, several blocks/slices]   gla_bwd_copy_rows: stage h0 and dht
//     [tokens]                           gla_bwd_local: chunk summaries of the state
//                                        and of its gradient (chained schedule: and
//                                        the scan itself, S_c, E_c and dh0)
//     [chained, staged dh0]              gla_bwd_copy_rows: dh0 back into place
//     [chained, packed, dh0 wanted]      gla_bwd_empty_dh0 for sequences without chunks
//     [separate scan: tokens or dh0]     gla_bwd_scan: S_c and E_c per chunk, dh0
//     [tokens]                           gla_bwd_chunk, gla_bwd_chunk_exact
//   [tokens, several shares]             gla_bwd_group_sum, gla_bwd_slice_sum,
//                                        gla_bwd_dv_sum
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gla.h"
#include "gla_internal.h"

namespace {

using gla::kChunk;
using gla::kVTile;

constexpr size_t kHeaderBytes = 256;  // status word + padding at the start of the workspace

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

// Keys of each launch: K itself up to 128, else two blocks (each a multiple of
// 16, at most 128).
int key_blocks(int K, int kb[2]) {
  if (K <= gla::kMaxKeyBlock) {
    kb[0] = K;
    kb[1] = 0;
    return 1;
  }
  kb[0] = ((K / 2 + 15) / 16) * 16;
  kb[1] = K - kb[0];
  return 2;
}

// The fast bf16 walker handles a problem whose keys fit one block.
bool uses_bf16_walker(const gla_problem *p) { return p->dtype == GLA_BF16 && p->K <= gla::kMaxKeyBlock; }

// Padded key width of the instantiation that runs a key block of kb keys.
int kernel_key_width(bool bf16_walker, bool bf16, int kb) {
  if (bf16_walker) return kb <= 64 ? 64 : 128;
  const int lo = bf16 ? 32 : 16;  // keys per contraction step of the general walker
  for (int w = lo; w <= 128; w *= 2)
    if (kb <= w) return w;
  return 128;
}

gla_status validate(const gla_problem *p) {
  if (!p) return GLA_ERR_NULL_ARG;
  if (p->B < 0 || p->T < 0 || p->H <= 0 || p->K <= 0 || p->V <= 0 || p->n_seqs < 0) return GLA_ERR_BAD_SHAPE;
  if (p->dtype != GLA_F32 && p->dtype != GLA_BF16) return GLA_ERR_BAD_DTYPE;
  if (!(std::isfinite(p->scale) && p->scale > 0.f)) return GLA_ERR_BAD_SCALE;
  if (p->chunk != kChunk) return GLA_ERR_UNSUPPORTED;
  if (p->K % 16 != 0 || p->K > 256 || p->V % 16 != 0 || p->V > 256) return GLA_ERR_UNSUPPORTED;
  if (p->value_tile != 0 && p->value_tile != 64 && p->value_tile != 128) return GLA_ERR_UNSUPPORTED;
  if (p->segment_chunks < 0 || (p->packed != 0 && p->packed != 1) || p->wait_limit < -1) return GLA_ERR_BAD_SHAPE;
  if (p->packed ? p->B != 1 : p->n_seqs != p->B) return GLA_ERR_BAD_SHAPE;
  if (p->HV < 0 || (p->HV != 0 && p->HV % p->H != 0)) return GLA_ERR_BAD_SHAPE;
  if (p->gate != GLA_GATE_PER_KEY && p->gate != GLA_GATE_PER_HEAD) return GLA_ERR_UNSUPPORTED;
  if (p->schedule < 0 || p->schedule > 3) return GLA_ERR_UNSUPPORTED;  // 3: the backward's walk
  // token-head rows and state elements must stay addressable with 64-bit
  // offsets; one chunk's byte range of any tensor (64 token rows of H heads)
  // must stay below 2^30, where the kernels put lanes with nothing to load
  const long long HV = p->HV == 0 ? p->H : p->HV;
  const double rows = (double)p->B * p->T * HV;
  if (rows * (p->K > p->V ? p->K : p->V) > 4.0e15) return GLA_ERR_BAD_SHAPE;
  if (HV * (p->K > p->V ? p->K : p->V) > (1LL << 22)) return GLA_ERR_BAD_SHAPE;
  return GLA_OK;
}

gla_status validate_fwd(const gla_problem *p) {
  const gla_status st = validate(p);
  if (st != GLA_OK) return st;
  return p->schedule == 3 ? GLA_ERR_UNSUPPORTED : GLA_OK;
}

// How the sequence axis is cut into state segments, and the workspace layout.
struct Plan {
  bool varlen;
  int N;          // sequences
  int R;          // chunks per segment
  int P;          // segments per sequence (fixed length)
  int seg_slots;  // upper bound on segments over all sequences
  int vtile;      // value columns per workgroup
  int NV;         // value slices per (segment, head)
  int nkb;        // key blocks
  int kb[2];      // keys per block
  bool segmented; // some sequence may span several segments
  bool fused;     // segments chained in one pass (gla_chunk_fused_bf16)
  long long units;
  size_t ws_state, ws_decay, ws_base, ws_opart, ws_link, ws_total;
  bool ok;        // index spaces fit the kernels' 32-bit grids
};

Plan make_plan(const gla_problem *p, bool varlen) {
  Plan pl{};
  pl.varlen = varlen;
  pl.N = varlen ? p->n_seqs : p->B;
  pl.nkb = key_blocks(p->K, pl.kb);
  const int H = p->HV == 0 ? p->H : p->HV;  // value heads: walkers, states and outputs count these
  const bool fast = uses_bf16_walker(p);
  // Value columns per workgroup.  The bf16 walker's 128-column workgroups form
  // the gated operands of a head once for all 128 columns; they are used when
  // they alone fill the device, or when sequences must be cut into segments
  // anyway.  Otherwise 64-column workgroups double the parallelism without
  // segmenting.  value_tile fixes the choice.
  int vtile = kVTile;
  if (fast) {
    const long long rows = (long long)pl.N * H;
    if (p->value_tile != 0) vtile = p->value_tile;
    else if (p->V % 128 != 0) vtile = 64;
    else if (varlen || rows * (p->V / 128) >= device_cu_count()) vtile = 128;
    else vtile = rows * (p->V / 64) >= device_cu_count() ? 64 : 128;
  }
  pl.vtile = vtile;
  pl.NV = (p->V + vtile - 1) / vtile;
  // one pass with chained segments (the bf16 walker with one key block): on
  // request, and by default for packed sequences, where its longer segments do
  // better than the three passes' shorter ones (16 sequences of U[256, 4096]
  // tokens: 224 against 250 us).  Fixed-length sequences default to three
  // passes: with one segment per compute unit every segment runs at once, and
  // the single pass's chain of start states costs what the scan launch saves
  // (B=1, H=32, T=65536: 998 against 987 us).
  const bool single = fast && (p->schedule == 2 || (p->schedule == 0 && varlen));
  const int NV = pl.NV;
  const long long chunks_total = ((long long)p->T + kChunk - 1) / kChunk;  // varlen: packed axis
  const long long chunks_seq = chunks_total;  // longest possible sequence
  long long R = p->segment_chunks;
  if (R == 0) {
    // Enough (segment, head, value slice) workgroups to give every compute
    // unit work; long sequences with few heads are cut into segments.  A
    // 128-column workgroup fills a compute unit on its own.
    const long long target = (vtile == 128 ? 1LL : 2LL) * device_cu_count();
    const long long units_one = (long long)pl.N * H * NV;
    if (!varlen) {
      if (units_one >= device_cu_count() || chunks_seq <= 1) {
        R = chunks_seq > 0 ? chunks_seq : 1;
      } else {
        long long P = (target + units_one - 1) / units_one;
        if (P > chunks_seq) P = chunks_seq;
        R = (chunks_seq + P - 1) / P;
      }
    } else {
      // packed: about 1.5 segment workgroups per compute unit balances the
      // unequal segment lengths (dispatched longest first) against the extra
      // summary work of cutting more sequences (measured optimum on the
      // 16-sequence U[256, 4096] workload)
      const long long work = (chunks_total + pl.N) * H * NV;  // chunk-slices to spread
      // one pass: about 2 workgroups per 3 compute units (fewer, longer
      // segments: each costs a walk start-up and a link in the chain; on the
      // same workload 48- to 52-chunk segments measured best, 221 us, against
      // 236 us at 42 to 47 and 258 us unsegmented)
      const long long tgt = single ? (2LL * device_cu_count()) / 3
                                   : vtile == 128 ? (3LL * device_cu_count()) / 2 : target;
      long long r = (work + tgt - 1) / tgt;
      if (r < 4) r = 4;
      R = r;
    }
    if (R < 1) R = 1;
  }
  if (R > INT_MAX) R = INT_MAX;
  pl.R = (int)R;
  long long slots;
  if (!varlen) {
    const long long P = chunks_seq <= 0 ? 1 : (chunks_seq + R - 1) / R;
    pl.P = P > INT_MAX ? INT_MAX : (int)P;
    slots = (long long)pl.N * P;
    pl.segmented = P > 1;
  } else {
    pl.P = 1;
    // every sequence has max(1, ceil(nc/R)) segments; nc <= len/64 + 1
    slots = pl.N + (chunks_total + pl.N + R - 1) / R;
    pl.segmented = chunks_total > R;  // a sequence needs more than one segment only if it has > R chunks
  }
  pl.seg_slots = slots > INT_MAX ? INT_MAX : (int)slots;
  pl.units = (pl.segmented ? slots : (long long)pl.N * (varlen ? 1 : pl.P)) * H;
  // grids: walker blocks = ceil(units / 8) * 8 * NV; scan blocks = N * H * ceil(K V / 1024)
  const long long walk_blocks = (pl.units + 7) / 8 * 8 * NV;
  const long long kmax = pl.kb[0] > pl.kb[1] ? pl.kb[0] : pl.kb[1];
  const long long scan_blocks = (long long)pl.N * H * ((kmax * p->V / 4 + 255) / 256);
  pl.ok = slots <= INT_MAX && pl.units <= INT_MAX && walk_blocks <= INT_MAX && scan_blocks <= INT_MAX;
  if (pl.segmented) {
    pl.ws_state = (size_t)slots * H * kmax * p->V * sizeof(float);
    pl.ws_decay = (size_t)slots * H * kmax * sizeof(float);
    pl.ws_base = varlen ? (size_t)(pl.N + 1 + slots) * sizeof(int32_t) : 0;  // table + order
  }
  if (pl.nkb == 2) pl.ws_opart = (size_t)p->B * p->T * H * p->V * sizeof(float);
  pl.fused = pl.segmented && fast && single;
  if (pl.fused) {
    pl.ws_link = (size_t)(1 + slots * H * NV) * sizeof(int32_t);  // counter + one flag per item
    pl.ok = pl.ok && 1 + slots * H * NV <= INT_MAX;
  }
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  pl.ws_total = kHeaderBytes + up(pl.ws_state) + up(pl.ws_decay) + up(pl.ws_base) + up(pl.ws_opart) + up(pl.ws_link);
  return pl;
}

// The launch sequence shared by the entry points: `workspace` holds at least
// plan.ws_total bytes, `status` is the word the kernels report into.
gla_status run_forward(const gla_problem *p, const Plan &pl, const void *q, const void *k, const void *v,
                       const float *g, const float *h0, const int32_t *cu_seqlens, void *o, float *ht,
                       char *ws, uint32_t *status, hipStream_t s) {
  const bool varlen = p->packed == 1;
  const int N = varlen ? p->n_seqs : p->B;
  if (N == 0) return GLA_OK;  // nothing to compute and no state to return
  if ((long long)p->B * p->T == 0 && ht == nullptr) return GLA_OK;
  const bool fast = uses_bf16_walker(p);
  const bool bf = p->dtype == GLA_BF16;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  gla::WalkParams w{};
  w.q = q; w.k = k; w.v = v; w.g = g; w.h0 = h0; w.cu = cu_seqlens; w.o = o; w.ht = ht;
  w.status = status;
  char *cur = ws + kHeaderBytes;
  w.seg_state = pl.segmented ? reinterpret_cast<float *>(cur) : nullptr;
  cur += up(pl.ws_state);
  w.seg_decay = pl.segmented ? reinterpret_cast<float *>(cur) : nullptr;
  cur += up(pl.ws_decay);
  int32_t *seg_base = (pl.segmented && varlen) ? reinterpret_cast<int32_t *>(cur) : nullptr;
  cur += up(pl.ws_base);
  float *o_part = pl.nkb == 2 ? reinterpret_cast<float *>(cur) : nullptr;
  cur += up(pl.ws_opart);
  w.link = pl.fused ? reinterpret_cast<int32_t *>(cur) : nullptr;
  w.seg_base = seg_base;
  w.seg_order = seg_base ? seg_base + N + 1 : nullptr;
  w.T = p->T; w.H = p->H; w.V = p->V; w.N = N;
  w.HV = p->HV == 0 ? p->H : p->HV;
  w.G = w.HV / p->H;
  w.gate_head = p->gate == GLA_GATE_PER_HEAD ? 1 : 0;
  w.Kmem = p->K;
  w.R = pl.R;
  w.P = pl.P;
  w.units = (int)pl.units;
  w.seg_slots = pl.seg_slots;
  w.vtile = pl.vtile;
  w.wait_polls = p->wait_limit == 0 ? gla::kDefaultWaitPolls : (p->wait_limit < 0 ? 0 : p->wait_limit);
  w.scale = p->scale;

  const long long nlink = (long long)(pl.ws_link / sizeof(int32_t));
  // packed sequences: the segment plan also zeroes the single pass's link table
  if (seg_base && gla::launch_segment_plan(w, seg_base, seg_base + N + 1, s, pl.fused ? w.link : nullptr,
                                           pl.fused ? (int)nlink : 0) != hipSuccess)
    return GLA_ERR_HIP;
  if (pl.fused) {  // one key block (the bf16 walker)
    w.K = pl.kb[0];
    w.koff = 0;
    if (!seg_base && gla::launch_clear(w.link, nlink, s) != hipSuccess) return GLA_ERR_HIP;
    if (gla::launch_fused_bf16(kernel_key_width(true, bf, w.K), w, s) != hipSuccess) return GLA_ERR_HIP;
    return GLA_OK;
  }
  int koff = 0;
  for (int b = 0; b < pl.nkb; ++b) {
    w.K = pl.kb[b];
    w.koff = koff;
    w.o_part = (pl.nkb == 2 && b == 0) ? o_part : nullptr;
    w.o_add = (pl.nkb == 2 && b == 1) ? o_part : nullptr;
    const int kd = kernel_key_width(fast, bf, w.K);
    auto walk = [&](bool local_mode) {
      return fast ? gla::launch_walk_bf16(local_mode, kd, w, s) : gla::launch_walk_general(local_mode, bf, kd, w, s);
    };
    if (pl.segmented) {
      if (walk(true) != hipSuccess) return GLA_ERR_HIP;
      if (gla::launch_state_scan(w, s) != hipSuccess) return GLA_ERR_HIP;
    }
    if (walk(false) != hipSuccess) return GLA_ERR_HIP;
    koff += w.K;
  }
  return GLA_OK;
}

// Backward: one chunk per slot (the forward's segment numbering with R = 1),
// and the backward's tables.  K past 128 is cut into two key blocks (as the
// forward's) and V into value slices of at most 128 columns; every (block,
// slice) runs one after another over the same state tables.
constexpr int kBwdSlice = 128;
int bwd_slices(int V) { return (V + kBwdSlice - 1) / kBwdSlice; }

struct BwdPlan {
  Plan fwd;  // slot numbering only (R = 1)
  int nkb, kb[2], slices;
  size_t off_base, off_fstate, off_dstate, off_ddecay, off_flags, off_dq_part, off_dk_part, off_dg_part, off_dv_part,
      off_bound, bound_bytes, off_chain_plan, off_plan_scratch, total;
  int cmax;  // packed: chunks of the longest possible sequence
  bool ok;
};

BwdPlan make_bwd_plan(const gla_problem *p, bool varlen) {
  BwdPlan b{};
  gla_problem p1 = *p;
  p1.segment_chunks = 1;
  b.fwd = make_plan(&p1, varlen);
  const Plan &pl = b.fwd;
  const long long HV = p->HV == 0 ? p->H : p->HV;
  const long long G = HV / p->H;
  const long long slots = pl.seg_slots;
  b.nkb = key_blocks(p->K, b.kb);
  b.slices = bwd_slices(p->V);
  const long long Kb = b.kb[0];                               // widest key block
  const long long Vs = p->V < kBwdSlice ? p->V : kBwdSlice;  // widest slice
  const bool gh = p->gate == GLA_GATE_PER_HEAD;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t cur = kHeaderBytes;
  b.off_base = cur;
  cur += up(varlen ? (size_t)(pl.N + 1 + slots) * sizeof(int32_t) : 0);
  b.off_fstate = cur;
  cur += up((size_t)slots * HV * Kb * Vs * sizeof(float));
  b.off_dstate = cur;
  cur += up((size_t)slots * HV * Kb * Vs * sizeof(float));
  b.off_ddecay = cur;
  cur += up((size_t)slots * HV * Kb * sizeof(float));
  b.off_flags = cur;
  cur += up((size_t)slots * HV * sizeof(int32_t));
  // fp32 shares: dq, dk per value head and slice; dg per slice (and key block,
  // with a per-head gate); dv per key block
  const size_t rows = (size_t)p->B * p->T;
  const size_t part = (G > 1 || b.slices > 1) ? up(b.slices * rows * HV * p->K * sizeof(float)) : 0;
  b.off_dq_part = cur;
  cur += part;
  b.off_dk_part = cur;
  cur += part;
  b.off_dg_part = cur;
  const int dg_parts = b.slices * (gh ? b.nkb : 1);
  cur += dg_parts > 1 ? up(dg_parts * rows * HV * (gh ? 1 : p->K) * sizeof(float)) : 0;
  b.off_dv_part = cur;
  cur += b.nkb > 1 ? up(b.nkb * rows * HV * p->V * sizeof(float)) : 0;
  // with several blocks or slices, the chained scan's h0, dht and dh0 rows and
  // columns of one (block, slice), staged compactly [N][HV][Kb][Vs]
  b.off_bound = cur;
  b.bound_bytes = up((size_t)pl.N * HV * Kb * Vs * sizeof(float));
  cur += (b.slices > 1 || b.nkb > 1) ? 3 * b.bound_bytes : 0;
  // packed: the chained scan's task table and its plan's scratch
  b.cmax = (int)(((long long)p->T + gla::kChunk - 1) / gla::kChunk);
  b.off_chain_plan = cur;
  cur += varlen ? up((size_t)gla::chain_plan_words(pl.seg_slots) * sizeof(int32_t)) : 0;
  b.off_plan_scratch = cur;
  cur += varlen ? up((size_t)gla::chain_plan_scratch_words(b.cmax, pl.N) * sizeof(int32_t)) : 0;
  b.total = cur;
  const long long scan_blocks = 2LL * pl.N * HV * ((Kb * Vs / 4 + 255) / 256);
  const long long rows_quads = (long long)p->B * p->T * p->H * (p->K / 4);
  // the chunk kernel addresses a chunk's 64 token rows of an output with
  // 32-bit byte offsets
  const long long row_bytes = 64LL * HV * (p->K > p->V ? p->K : p->V) * 4;
  b.ok = pl.ok && 2 * slots * HV <= INT_MAX && scan_blocks <= INT_MAX && (rows_quads + 255) / 256 <= INT_MAX &&
         row_bytes <= INT_MAX;
  return b;
}

// Whether the backward walks its chains (schedule 0), for N sequences with HV
// value heads; else it runs the separate scan.  The walk takes one workgroup
// per chain (2 N HV of them) and moves no state but the stores; with fewer
// chains than half the compute units the chains, one chunk at a time, set the
// pace.  Measured on MI355X, K = V = 128 bf16, us for the separate scan /
// chained scan / walk (N HV pairs, chunks per sequence):
//   128 pairs, 32 chunks  1011 / 861 / 709      512 pairs, 8 chunks  972 / 824 / 724
//    64 pairs, 64 chunks   991 / 966 / 920       64 pairs, 32 chunks 511 / 514 / 478
//    32 pairs, 32 chunks   246 / 339 / 348       16 pairs, 128 chunks 520 / 935 / 1130
// The chained scan is never faster than both others; it stays as schedule 2.
bool bwd_walk_pays(long long N, long long HV) { return 4 * N * HV >= device_cu_count(); }

gla_status validate_bwd(const gla_problem *p) {
  const gla_status st = validate(p);
  if (st != GLA_OK) return st;
  return GLA_OK;
}

gla_status run_backward(const gla_problem *p, const BwdPlan &bpl, const void *q, const void *k, const void *v,
                        const float *g, const float *h0, const int32_t *cu_seqlens, const void *dout,
                        const float *dht, void *dq, void *dk, void *dv, float *dg, float *dh0, char *ws,
                        uint32_t *status, hipStream_t s) {
  const bool varlen = p->packed == 1;
  const int N = varlen ? p->n_seqs : p->B;
  if (N == 0) return GLA_OK;
  const bool tokens = (long long)p->B * p->T > 0;
  if (!tokens && dh0 == nullptr) return GLA_OK;
  const Plan &pl = bpl.fwd;
  const bool bf = p->dtype == GLA_BF16;
  gla::WalkParams w{};
  w.q = q; w.k = k; w.v = v; w.g = g; w.h0 = h0; w.cu = cu_seqlens;
  w.status = status;
  int32_t *seg_base = varlen ? reinterpret_cast<int32_t *>(ws + bpl.off_base) : nullptr;
  w.seg_base = seg_base;
  w.T = p->T; w.H = p->H; w.K = p->K; w.V = p->V; w.N = N;
  w.HV = p->HV == 0 ? p->H : p->HV;
  w.G = w.HV / p->H;
  w.gate_head = p->gate == GLA_GATE_PER_HEAD ? 1 : 0;
  w.Kmem = p->K;
  w.R = pl.R;
  w.P = pl.P;
  w.seg_slots = pl.seg_slots;
  w.scale = p->scale;
  w.wait_polls = p->wait_limit == 0 ? gla::kDefaultWaitPolls : (p->wait_limit < 0 ? 0 : p->wait_limit);
  if (seg_base && gla::launch_segment_plan(w, seg_base, seg_base + N + 1, s) != hipSuccess) return GLA_ERR_HIP;
  gla::BwdParams b{};
  b.w = w;  // seg_order stays null: the backward's kernels take slots in plain order
  b.persistent_blocks = 2 * device_cu_count();
  b.Vmem = p->V;
  b.fstate = reinterpret_cast<float *>(ws + bpl.off_fstate);
  b.dstate = reinterpret_cast<float *>(ws + bpl.off_dstate);
  b.ddecay = reinterpret_cast<float *>(ws + bpl.off_ddecay);
  b.flags = reinterpret_cast<int32_t *>(ws + bpl.off_flags);
  const int slices = bpl.slices, nkb = bpl.nkb;
  const bool gh = w.gate_head != 0;
  const long long rows = (long long)p->B * p->T;
  float *dq_part = nullptr, *dk_part = nullptr;
  if (w.G > 1 || slices > 1) {
    dq_part = reinterpret_cast<float *>(ws + bpl.off_dq_part);
    dk_part = reinterpret_cast<float *>(ws + bpl.off_dk_part);
  }
  const int dg_nparts = slices * (gh ? nkb : 1);
  float *dg_parts = dg_nparts > 1 ? reinterpret_cast<float *>(ws + bpl.off_dg_part) : nullptr;
  float *dv_parts = nkb > 1 ? reinterpret_cast<float *>(ws + bpl.off_dv_part) : nullptr;
  const long long dg_share = rows * w.HV * (gh ? 1 : p->K), dv_share = rows * w.HV * p->V;
  // The scan can run inside the summary kernel (one chain per sequence, value
  // head and direction): chained, the chains' tasks spread over all
  // workgroups and meet through links in memory; walked, each workgroup
  // carries one chain's state from chunk to chunk.  Both save the scan's pass
  // over both state tables.
  const long long tasks = 2LL * pl.seg_slots * w.HV;
  const bool walk = tokens && (p->schedule == 3 || (p->schedule == 0 && bwd_walk_pays(N, w.HV)));
  const bool chained = tokens && !walk && p->schedule == 2 && tasks + b.persistent_blocks <= INT_MAX;
  b.walk = walk ? 1 : 0;
  if ((chained || walk) && varlen) {
    // packed: the task table orders each step's chains by sequence length
    b.chain_plan = reinterpret_cast<int32_t *>(ws + bpl.off_chain_plan);
    if (gla::launch_chain_plan(b, bpl.cmax, reinterpret_cast<int32_t *>(ws + bpl.off_plan_scratch), s) !=
        hipSuccess)
      return GLA_ERR_HIP;
  }
  // the chained scan's link takes h0, dht and dh0 as [N][HV][Kb][Vs] of its
  // block and slice: with several of either they are staged through the
  // workspace (groups of Kb rows, one group per sequence and value head)
  const bool stage = (chained || walk) && (slices > 1 || nkb > 1);
  float *stage_h0 = reinterpret_cast<float *>(ws + bpl.off_bound);
  float *stage_dht = reinterpret_cast<float *>(ws + bpl.off_bound + bpl.bound_bytes);
  float *stage_dh0 = reinterpret_cast<float *>(ws + bpl.off_bound + 2 * bpl.bound_bytes);
  const long long groups = (long long)N * w.HV;
  const long long full_group = (long long)p->K * p->V;  // one state of h0, dht, dh0
  const size_t es = bf ? 2 : 4;
  // Each (key block, value slice) runs the whole sequence of launches over the
  // same state tables (stream order keeps one's tables until its chunk kernel
  // is done).
  for (int kbi = 0; kbi < nkb; ++kbi) {
    const int koff = kbi == 0 ? 0 : bpl.kb[0];
    b.w.K = bpl.kb[kbi];
    b.w.Kmem = p->K;
    b.w.q = static_cast<const char *>(q) + koff * es;
    b.w.k = static_cast<const char *>(k) + koff * es;
    b.w.g = gh ? g : g + koff;
    b.dq = static_cast<char *>(dq) + koff * es;
    b.dk = static_cast<char *>(dk) + koff * es;
    for (int sl = 0; sl < slices; ++sl) {
      const int voff = sl * kBwdSlice;
      b.w.V = p->V - voff < kBwdSlice ? p->V - voff : kBwdSlice;
      const long long boff = (long long)koff * p->V + voff;  // first element of h0, dht, dh0
      b.w.v = static_cast<const char *>(v) + voff * es;
      b.w.h0 = h0 ? h0 + boff : nullptr;
      b.dout = static_cast<const char *>(dout) + voff * es;
      b.dv = static_cast<char *>(dv) + voff * es;
      b.dv_part = dv_parts ? dv_parts + kbi * dv_share + voff : nullptr;
      b.dht = dht ? dht + boff : nullptr;
      b.dh0 = dh0 ? dh0 + boff : nullptr;
      b.dq_part = dq_part ? dq_part + sl * rows * w.HV * p->K + koff : nullptr;
      b.dk_part = dk_part ? dk_part + sl * rows * w.HV * p->K + koff : nullptr;
      if (dg_parts) b.dg = dg_parts + (gh ? (long long)(kbi * slices + sl) : sl) * dg_share + (gh ? 0 : koff);
      else b.dg = gh ? dg : dg + koff;
      b.chain = nullptr;
      if (chained) {
        // the decay table is only read by gla_bwd_scan, which this schedule
        // does not launch: it holds the chains' counter and flags instead
        b.chain = reinterpret_cast<int32_t *>(ws + bpl.off_ddecay);
        if (gla::launch_clear(b.chain, 1 + tasks, s) != hipSuccess) return GLA_ERR_HIP;
      }
      const long long cg = (long long)b.w.K * b.w.V;  // one compact state
      if (stage) {
        if (h0) {
          if (gla::launch_copy_rows(stage_h0, cg, b.w.V, b.w.h0, full_group, p->V, groups, b.w.K, b.w.V, s) !=
              hipSuccess)
            return GLA_ERR_HIP;
          b.w.h0 = stage_h0;
        }
        if (dht) {
          if (gla::launch_copy_rows(stage_dht, cg, b.w.V, b.dht, full_group, p->V, groups, b.w.K, b.w.V, s) !=
              hipSuccess)
            return GLA_ERR_HIP;
          b.dht = stage_dht;
        }
        if (dh0) b.dh0 = stage_dh0;
      }
      if (tokens && gla::launch_bwd_local(bf, b, s) != hipSuccess) return GLA_ERR_HIP;
      if (stage && dh0 &&
          gla::launch_copy_rows(dh0 + boff, full_group, p->V, stage_dh0, cg, b.w.V, groups, b.w.K, b.w.V, s) !=
              hipSuccess)
        return GLA_ERR_HIP;
      if ((chained || walk) && varlen && dh0) {
        // sequences without chunks have no chain: their dh0 is dht (or zero)
        gla::BwdParams e = b;
        e.dh0 = dh0 + boff;
        e.dht = dht ? dht + boff : nullptr;
        if (gla::launch_empty_dh0(e, s) != hipSuccess) return GLA_ERR_HIP;
      }
      if (!chained && !walk && gla::launch_bwd_scan(b, s) != hipSuccess) return GLA_ERR_HIP;
      if (tokens && gla::launch_bwd_chunk(bf, b, s) != hipSuccess) return GLA_ERR_HIP;
    }
  }
  if (tokens) {
    b.w.K = p->K;  // the shares hold rows of all keys
    b.dq = dq;
    b.dk = dk;
    b.dq_part = dq_part;
    b.dk_part = dk_part;
    if (gla::launch_bwd_finish(bf, b, slices, dg_parts, dg_nparts, dg, s) != hipSuccess) return GLA_ERR_HIP;
    if (dv_parts && gla::launch_dv_sum(bf, dv, dv_parts, dv_share, nkb, s) != hipSuccess) return GLA_ERR_HIP;
  }
  return GLA_OK;
}

// WY-representation forward: one chunk per slot, the slot table of packed
// inputs in the workspace after the status header.
struct WyPlan {
  Plan fwd;  // slot numbering (R = 1)
  size_t total;
  bool ok;
};

gla_problem wy_as_problem(const gla_wy_problem *p) {
  gla_problem q{};
  q.B = p->B; q.T = p->T; q.H = p->H; q.K = p->K; q.V = p->V; q.dtype = p->dtype;
  q.n_seqs = p->n_seqs; q.chunk = p->chunk; q.scale = 1.f; q.segment_chunks = 1; q.packed = p->packed;
  q.HV = p->HV;
  return q;
}

gla_status validate_wy(const gla_wy_problem *p) {
  if (!p) return GLA_ERR_NULL_ARG;
  const gla_problem q = wy_as_problem(p);
  return validate(&q);
}

WyPlan make_wy_plan(const gla_wy_problem *p) {
  WyPlan w{};
  const gla_problem q = wy_as_problem(p);
  w.fwd = make_plan(&q, p->packed == 1);
  const long long HV = p->HV == 0 ? p->H : p->HV;
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  w.total = kHeaderBytes + up(p->packed == 1 ? (size_t)(w.fwd.N + 1 + w.fwd.seg_slots) * sizeof(int32_t) : 0);
  w.ok = w.fwd.ok && (long long)w.fwd.seg_slots * HV <= INT_MAX;
  return w;
}

// Host-side checks of a call (same for both entry points).
gla_status check_call(const gla_problem *p, const void *q, const void *k, const void *v, const float *g,
                      const void *o, const int32_t *cu_seqlens, Plan &pl) {
  gla_status st = validate_fwd(p);
  if (st != GLA_OK) return st;
  const bool varlen = p->packed == 1;
  if (varlen != (cu_seqlens != nullptr)) return GLA_ERR_NULL_ARG;
  const bool empty_tokens = (long long)p->B * p->T == 0;
  if (!empty_tokens && (!q || !k || !v || !g || !o)) return GLA_ERR_NULL_ARG;
  pl = make_plan(p, varlen);
  if (!pl.ok) return GLA_ERR_BAD_SHAPE;
  return GLA_OK;
}

// Scratch of gla_fwd_noalloc: one array per device, resident until the process
// ends.  Host code never uses the array's name as an address (on the host it
// is a stand-in, not device memory): each device's address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

char *scratch_for_current_device() {
  static std::mutex mu;
  static char *addr[64] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    addr[dev] = reinterpret_cast<char *>(ptr);
  }
  return addr[dev];
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
    case GLA_ERR_UNSUPPORTED: return "unsupported K, V, chunk or value tile (backward: K, V <= 128)";
    case GLA_ERR_WORKSPACE: return "workspace missing or too small";
    case GLA_ERR_HIP: return "HIP runtime or launch failure";
  }
  return "unknown status";
}

size_t gla_fwd_workspace_bytes(const gla_problem *p) {
  if (validate_fwd(p) != GLA_OK) return (size_t)-1;
  const Plan pl = make_plan(p, p->packed == 1);
  if (!pl.ok) return (size_t)-1;
  return pl.ws_total;
}

gla_status gla_fwd(const gla_problem *p, const void *q, const void *k, const void *v, const float *g,
                   const float *h0, const int32_t *cu_seqlens, void *o, float *ht, void *workspace,
                   size_t workspace_bytes, void *stream) {
  Plan pl;
  const gla_status st = check_call(p, q, k, v, g, o, cu_seqlens, pl);
  if (st != GLA_OK) return st;
  if (workspace == nullptr || workspace_bytes < pl.ws_total) return GLA_ERR_WORKSPACE;
  char *ws = reinterpret_cast<char *>(workspace);
  return run_forward(p, pl, q, k, v, g, h0, cu_seqlens, o, ht, ws, reinterpret_cast<uint32_t *>(ws),
                     reinterpret_cast<hipStream_t>(stream));
}

size_t gla_bwd_workspace_bytes(const gla_problem *p) {
  if (validate_bwd(p) != GLA_OK) return (size_t)-1;
  const BwdPlan b = make_bwd_plan(p, p->packed == 1);
  if (!b.ok) return (size_t)-1;
  return b.total;
}

gla_status gla_bwd(const gla_problem *p, const void *q, const void *k, const void *v, const float *g,
                   const float *h0, const int32_t *cu_seqlens, const void *dout, const float *dht, void *dq,
                   void *dk, void *dv, float *dg, float *dh0, void *workspace, size_t workspace_bytes,
                   void *stream) {
  const gla_status st = validate_bwd(p);
  if (st != GLA_OK) return st;
  const bool varlen = p->packed == 1;
  if (varlen != (cu_seqlens != nullptr)) return GLA_ERR_NULL_ARG;
  const bool empty_tokens = (long long)p->B * p->T == 0;
  if (!empty_tokens && (!q || !k || !v || !g || !dout || !dq || !dk || !dv || !dg)) return GLA_ERR_NULL_ARG;
  const BwdPlan b = make_bwd_plan(p, varlen);
  if (!b.ok) return GLA_ERR_BAD_SHAPE;
  if (workspace == nullptr || workspace_bytes < b.total) return GLA_ERR_WORKSPACE;
  char *ws = reinterpret_cast<char *>(workspace);
  return run_backward(p, b, q, k, v, g, h0, cu_seqlens, dout, dht, dq, dk, dv, dg, dh0, ws,
                      reinterpret_cast<uint32_t *>(ws), reinterpret_cast<hipStream_t>(stream));
}

size_t gla_wy_fwd_workspace_bytes(const gla_wy_problem *p) {
  if (validate_wy(p) != GLA_OK) return (size_t)-1;
  const WyPlan w = make_wy_plan(p);
  return w.ok ? w.total : (size_t)-1;
}

gla_status gla_wy_fwd(const gla_wy_problem *p, const void *k, const void *v, const float *beta, const void *A,
                      const float *g, const int32_t *cu_seqlens, void *w, void *u, void *workspace,
                      size_t workspace_bytes, void *stream) {
  const gla_status st = validate_wy(p);
  if (st != GLA_OK) return st;
  const bool varlen = p->packed == 1;
  if (varlen != (cu_seqlens != nullptr)) return GLA_ERR_NULL_ARG;
  if ((long long)p->B * p->T > 0 && (!k || !v || !beta || !A || !w || !u)) return GLA_ERR_NULL_ARG;
  const WyPlan pl = make_wy_plan(p);
  if (!pl.ok) return GLA_ERR_BAD_SHAPE;
  if (workspace == nullptr || workspace_bytes < pl.total) return GLA_ERR_WORKSPACE;
  const int N = varlen ? p->n_seqs : p->B;
  if (N == 0 || (long long)p->B * p->T == 0) return GLA_OK;
  char *ws = reinterpret_cast<char *>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  gla::WyParams wp{};
  gla::WalkParams &wk = wp.w;
  wk.k = k; wk.v = v; wk.cu = cu_seqlens;
  wk.status = reinterpret_cast<uint32_t *>(ws);
  int32_t *seg_base = varlen ? reinterpret_cast<int32_t *>(ws + kHeaderBytes) : nullptr;
  wk.seg_base = seg_base;
  wk.T = p->T; wk.H = p->H; wk.K = p->K; wk.V = p->V; wk.N = N;
  wk.HV = p->HV == 0 ? p->H : p->HV;
  wk.G = wk.HV / p->H;
  wk.Kmem = p->K;
  wk.R = pl.fwd.R;
  wk.P = pl.fwd.P;
  wk.seg_slots = pl.fwd.seg_slots;
  wp.beta = beta; wp.A = A; wp.g = g; wp.wout = w; wp.u = u;
  if (seg_base && gla::launch_segment_plan(wk, seg_base, seg_base + N + 1, s) != hipSuccess) return GLA_ERR_HIP;
  if (gla::launch_wy_fwd(p->dtype == GLA_BF16, wp, s) != hipSuccess) return GLA_ERR_HIP;
  return GLA_OK;
}

gla_status gla_fwd_noalloc(const gla_problem *p, const void *q, const void *k, const void *v, const float *g,
                           const float *h0, const int32_t *cu_seqlens, void *o, float *ht, uint32_t *status,
                           void *stream) {
  Plan pl;
  const gla_status st = check_call(p, q, k, v, g, o, cu_seqlens, pl);
  if (st != GLA_OK) return st;
  if (pl.ws_total > kScratchBytes) return GLA_ERR_WORKSPACE;
  char *ws = scratch_for_current_device();
  if (ws == nullptr) return GLA_ERR_HIP;
  // without a caller word, reports go to the scratch header, which nobody reads
  return run_forward(p, pl, q, k, v, g, h0, cu_seqlens, o, ht, ws,
                     status != nullptr ? status : reinterpret_cast<uint32_t *>(ws),
                     reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"
