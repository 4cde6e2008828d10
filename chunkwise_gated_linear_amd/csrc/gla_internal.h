// Internal interface between the host library (gla_host.hip) and the device
// kernels (gla_kernels.hip, gla_walk_bf16.hip, gla_bwd.hip, gla_wy.hip).  Not
// part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

constexpr int kChunk = 64;     // tokens per chunk
constexpr int kVTile = 64;     // value columns handled by one general-walker workgroup
constexpr int kThreads = 256;  // threads per general-walker workgroup (4 waves of 64)
constexpr int kMaxKeyBlock = 128;  // keys one launch handles; wider K is cut into key blocks
constexpr int kDefaultWaitPolls = 1 << 22;
// Smallest decay of one key over one chunk (exp of its summed log decay) that
// the factorised in-chunk form holds in fp32: its factors reach 1 / decay.
// Chunks below it are evaluated token by token (e^-80).
constexpr float kMinChunkDecay = 1.80485139e-35f;
constexpr float kMinChunkLogDecay = -80.f;  // the same bound on the summed log decay

// Everything a launch needs; passed by value as the kernel argument.
//
// Key blocks: one launch covers keys [koff, koff + K) of the Kmem keys per head
// in q, k, g, h0 and ht.  Every key row of the state evolves on its own, so the
// output is the sum of the key blocks' outputs: with two blocks the first writes
// its fp32 partial output to o_part, the second adds o_add (= that partial)
// before rounding and storing o.
//
// Heads: q and k have H key heads; v, g, o, h0, ht and every state have HV value
// heads (HV = G H), and value head hv reads key head hv / G.  Walkers, segments
// and units count value heads.
struct WalkParams {
  const void *q, *k, *v;       // [B,T,H,Kmem] / [B,T,HV,V], dtype per instantiation
  const float *g;              // [B,T,HV,Kmem] (a decay per key) or [B,T,HV] (gate_head)
  const float *h0;             // [N,HV,Kmem,V] or null
  const int32_t *cu;           // [N+1] or null
  void *o;                     // [B,T,HV,V]
  float *ht;                   // [N,HV,Kmem,V] or null
  float *seg_state;            // [seg_slots][HV][K][V]: segment summaries, then start states
  float *seg_decay;            // [seg_slots][HV][K]: product of the segment's decays
  const int32_t *seg_base;     // [N+1] first segment of each packed sequence, or null
  const int32_t *seg_order;    // [seg_slots] segment ids, longest first (packed), or null
  uint32_t *status;            // sticky status word (GLA_STATUS_* bits)
  int32_t *link;               // single pass: [0] item counter, then one flag per (slot, HV, value slice); zeroed before the launch
  float *o_part;               // [B,T,HV,V] fp32: write the partial output here instead of o, or null
  const float *o_add;          // [B,T,HV,V] fp32: partial output of the other key block, or null
  int32_t T, H, K, V, N;       // H: key heads; K: keys of this launch's block
  int32_t HV, G;               // value heads, value heads per key head
  int32_t gate_head;           // 1: one decay per value head and token, g [B,T,HV]
  int32_t Kmem;                // keys per head in memory (row stride of q, k, g, h0, ht)
  int32_t koff;                // first key of this launch's block
  int32_t R;                   // chunks per segment
  int32_t P;                   // segments per sequence when seg_base is null
  int32_t units;               // (segment, value head) pairs covered by the grid
  int32_t seg_slots;           // segment slots the workspace holds
  int32_t vtile;               // value columns per workgroup (64, or 128 for the bf16 walker)
  int32_t wait_polls;          // bound on each wait between waves (0: none, report at once)
  float scale;
};

// Launchers (return the hipGetLastError() of the launch).
// The general walker (gla_kernels.hip): fp32 any key block, bf16 key blocks of a
// split K; kd is the padded key width of the instantiation (16, 32, 64, 128).
hipError_t launch_walk_general(bool local_mode, bool bf16, int kd, const WalkParams &p, hipStream_t s);
hipError_t launch_state_scan(const WalkParams &p, hipStream_t s);
// The segment table of packed sequences; it also zeroes `nclear` words at
// `clear` (the single pass's link table), or none.
hipError_t launch_segment_plan(const WalkParams &p, int32_t *seg_base, int32_t *seg_order, hipStream_t s,
                               int32_t *clear = nullptr, int nclear = 0);
// bf16 walker (gla_walk_bf16.hip): key widths kd in {64, 128} (a narrower key
// block is padded with zero keys), 64 or 128 value columns per workgroup
// (WalkParams::vtile), any V (columns past V are masked)
hipError_t launch_walk_bf16(bool local_mode, int kd, const WalkParams &p, hipStream_t s);
// The single pass (summary, scan and outputs in one launch) of the bf16 walker;
// needs seg_state, seg_decay and a zeroed link table.
hipError_t launch_fused_bf16(int kd, const WalkParams &p, hipStream_t s);
// Zeroes n 32-bit words (a kernel, not a memset node, so callers may capture it).
hipError_t launch_clear(int32_t *words, long long n, hipStream_t s);

// Backward (gla_bwd.hip).  The state tables hold one chunk per slot: chunk c
// of sequence n is slot first(n) + c, with first(n) = n P (fixed length) or
// seg_base[n] (packed), as the forward kernels number segments of one chunk
// (gla_segment_plan with R = 1 fills seg_base).  K past 128 is cut into two
// key blocks and V past 128 into value slices of at most 128 columns; each
// (block, slice) is launched on its own: w.K / w.V the block's keys and the
// slice's columns, the tensors offset to their first key and column, w.Kmem
// and Vmem the full widths (the row strides).
// words of the chain plan: the chained schedule's task count, the number of
// sequences with chunks, the table
constexpr int kChainPlanTasks = 0, kChainPlanSeqs = 1, kChainPlanTable = 2;
constexpr int chain_plan_words(int slots) { return kChainPlanTable + 2 * slots; }
// scratch words of launch_chain_plan for sequences of at most cmax chunks
constexpr long long chain_plan_scratch_words(int cmax, int N) { return 3LL * cmax + 4 + N; }

struct BwdParams {
  WalkParams w;          // problem sizes, q, k, v, g, h0, cu, seg_base (seg_order null), scale
  const void *dout;      // [B,T,HV,V] dtype: gradient of o
  const float *dht;      // [N,HV,K,V] gradient of ht, or null (zero)
  void *dq, *dk;         // [B,T,H,K] dtype
  void *dv;              // [B,T,HV,V] dtype
  float *dg;             // [B,T,HV,K], or [B,T,HV] with a per-head gate
  float *dh0;            // [N,HV,K,V] or null
  float *fstate;         // [slots][HV][K][V]: chunk summaries of the state, then S_c (state before chunk c)
  float *dstate;         // [slots][HV][K][V]: chunk summaries of the state gradient, then E_c
  float *ddecay;         // [slots][HV][K]: e^{G_last} of each chunk
  int32_t *chain;        // the chained schedule, or null: gla_bwd_local also walks the chains
                         // of S_c and E_c ([0] task counter, then flags [2][slots][HV]; zeroed
                         // before the launch) and gla_bwd_scan is not launched.  Its h0, dht and
                         // dh0 are [N][HV][K][V] (a value slice's columns staged compactly)
  int32_t *chain_plan;   // packed sequences, chained or walk: [kChainPlanTasks] task count,
                         // [kChainPlanSeqs] sequences with chunks, from word kChainPlanTable
                         // the (step, sequence) int2 table (launch_chain_plan)
  int32_t *flags;        // [slots][HV]: 1 when the chunk is left to the token-by-token kernel
  float *dq_part, *dk_part;  // [B,T,HV,Kmem] fp32 shares of dq, dk of this value slice (G > 1 or several slices), else null
  float *dv_part;            // [B,T,HV,Vmem] fp32 share of dv of this key block (several key blocks), else null
  int32_t Vmem;              // value columns per row of v, do, dv, h0, dht, dh0
  int32_t persistent_blocks; // workgroups of the persistent kernels (a few per compute unit)
  int32_t walk;              // 1: the walk schedule (read by the launcher only): each workgroup of
                             // gla_bwd_local walks whole chains of S_c / E_c, carrying the state
                             // (h0, dht, dh0 laid out as for the chained schedule; no counter
                             // or flags), and gla_bwd_scan is not launched
};
hipError_t launch_bwd_local(bool bf16, const BwdParams &bp, hipStream_t s);
hipError_t launch_bwd_scan(const BwdParams &bp, hipStream_t s);
// the fast chunk kernel and the token-by-token kernel for flagged chunks
hipError_t launch_bwd_chunk(bool bf16, const BwdParams &bp, hipStream_t s);
// After every key block and value slice: with dq_part, dq and dk as the sums
// of the shares over value heads and `slices` slices (bp.dq_part / dk_part at
// slice 0, rows of bp.w.K keys); with dg_nparts > 1, dg as the sum of the
// shares dg_parts.
hipError_t launch_bwd_finish(bool bf16, const BwdParams &bp, int slices, const float *dg_parts, int dg_nparts,
                             float *dg, hipStream_t s);
// Columns [0, cols) of groups x rows fp32 rows: row r of group gi from src +
// gi src_group + r src_row to dst + gi dst_group + r dst_row; cols, strides
// and bases multiples of 4 floats.
hipError_t launch_copy_rows(float *dst, int64_t dst_group, int64_t dst_row, const float *src, int64_t src_group,
                            int64_t src_row, long long groups, int rows, int cols, hipStream_t s);
// The chained scan's task table for packed sequences (bp.chain_plan, from
// cu_seqlens; sequences of at most cmax chunks; scratch of
// chain_plan_scratch_words(cmax, N) words).
hipError_t launch_chain_plan(const BwdParams &bp, int cmax, int32_t *scratch, hipStream_t s);
// dh0 = dht (or zero) for the packed sequences without chunks.
hipError_t launch_empty_dh0(const BwdParams &bp, hipStream_t s);
// dv (n elements, input dtype) = the sum of `blocks` fp32 shares n apart.
hipError_t launch_dv_sum(bool bf16, void *dv, const float *parts, long long n, int blocks, hipStream_t s);

// WY-representation forward (gla_wy.hip): one chunk per slot as in the backward.
struct WyParams {
  WalkParams w;        // sizes (T, H, HV, G, K, V, N, P, seg_slots), k = w.k, v = w.v, cu, seg_base
  const float *beta;   // [B,T,HV]
  const void *A;       // [B,T,HV,64] dtype: each token's row of its chunk matrix
  const float *g;      // [B,T,HV] base-2 log gate, or null
  void *wout;          // [B,T,HV,K] dtype
  void *u;             // [B,T,HV,V] dtype
};
hipError_t launch_wy_fwd(bool bf16, const WyParams &wp, hipStream_t s);

}  // namespace gla
