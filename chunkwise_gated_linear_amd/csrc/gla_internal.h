// Internal interface between the host library (gla_host.hip) and the device
// kernels (gla_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

constexpr int kChunk = 64;     // tokens per chunk
constexpr int kVTile = 64;     // value columns handled by one workgroup
constexpr int kThreads = 256;  // threads per walker workgroup (4 waves of 64)

// Everything a launch needs; passed by value as the kernel argument.
struct WalkParams {
  const void *q, *k, *v;       // [B,T,H,K] / [B,T,H,V], dtype per instantiation
  const float *g;              // [B,T,H,K]
  const float *h0;             // [N,H,K,V] or null
  const int32_t *cu;           // [N+1] or null
  void *o;                     // [B,T,H,V]
  float *ht;                   // [N,H,K,V] or null
  float *seg_state;            // [seg_slots][H][K][V]: segment summaries, then start states
  float *seg_decay;            // [seg_slots][H][K]: product of the segment's decays
  const int32_t *seg_base;     // [N+1] first segment of each packed sequence, or null
  const int32_t *seg_order;    // [segments] segment ids, longest first (packed), or null
  int32_t T, H, K, V, N;
  int32_t R;                   // chunks per segment
  int32_t P;                   // segments per sequence when seg_base is null
  int32_t units;               // (segment, head) pairs covered by the grid
  int32_t vtile;               // value columns per workgroup (64, or 128 for the bf16 walker)
  float scale;
};

// Launchers (return the hipGetLastError() of the launch).
hipError_t launch_walk(bool local_mode, bool bf16, int K, const WalkParams &p, hipStream_t s);
hipError_t launch_state_scan(const WalkParams &p, hipStream_t s);
// bf16 walker for K in {64, 128} (gla_walk_bf16.hip), 64 or 128 value columns
// per workgroup (WalkParams::vtile)
bool walk_bf16_supported(int K);
hipError_t launch_walk_bf16(bool local_mode, int K, const WalkParams &p, hipStream_t s);
// whether launch_walk runs the bf16 walker for this dtype and K
bool bf16_walker_used(bool bf16, int K);
hipError_t launch_segment_plan(const WalkParams &p, int32_t *seg_base, int32_t *seg_order, hipStream_t s);

}  // namespace gla
