// Internal declarations of the gfx950 Fathom library (kernels + launchers).
// Not part of the public ABI; see include/fathom.h for the calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fathom.h"

namespace fathom {

constexpr int kBlock = 64;   // tokens per block = bits per plane word = wave64 lanes
constexpr int kPlanes = 4;   // bit planes of the 4-bit code
constexpr int kD = 128;      // channels per KV head supported by the kernels

// Launchers: enqueue on `stream`, return the hipError_t of the launch.
hipError_t launch_encode(const uint16_t* k, int64_t groups, int64_t n, int64_t nb_store,
                         int64_t block_offset, uint64_t* planes, uint16_t* scales,
                         uint32_t* nonfinite_flag, hipStream_t stream);

// fathom_append_plan: launch_encode and launch_plan in one launch when the
// append is at most 64 blocks per group (else the two launches).
hipError_t launch_append_plan(const uint16_t* k, int64_t groups, int64_t n, int64_t nb_store,
                              int64_t block_offset, uint64_t* planes, uint16_t* scales,
                              uint32_t* nonfinite_flag, const float* q, const float* var, int G,
                              int budget_bits, uint8_t* depths, double* theta,
                              int32_t* bits_used, hipStream_t stream);
hipError_t launch_plan(const float* q, const float* var, int64_t groups, int G,
                       int budget_bits, uint8_t* depths, double* theta, int32_t* bits_used,
                       hipStream_t stream);

hipError_t launch_plan_fixed(const float* q, const float* stat, int64_t groups, int G, int mode,
                             int param, uint8_t* depths, hipStream_t stream);
// ev_start / ev_stop (may be null): recorded from the first and the last
// kernel's own start and end timestamps.
hipError_t launch_scan(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                       const uint8_t* depths, const float* q, int64_t groups, int G,
                       int64_t n, float* scores, hipStream_t stream,
                       hipEvent_t ev_start = nullptr, hipEvent_t ev_stop = nullptr);

// Workgroups fathom_scan launches for `groups` groups of n keys.
int64_t scan_max_workgroups(int64_t groups, int64_t n);

size_t topk_workspace_bytes(int64_t rows, int64_t n, int k);
// Pieces of fathom_scan_topk's selection (workspace layout: topk::FusedWs).
// fathom_test_cut_hooks: whether the candidate scan (set_cut_hooks) and
// fathom_topk's cut workgroups (set_topk_cut_hooks) publish their cuts, and
// the poll limit of the waves that wait for them (defaults 1 and 2048).
void set_cut_hooks(int publish, int spin_limit);
void set_topk_cut_hooks(int publish, int spin_limit);

// Chunks [0, npacked) of a row come in runs of `pack` whose candidates are
// packed from the run's first slot (1 and 0: every chunk on its own).
hipError_t launch_fused_resolve(const float* scores, int64_t rows, int64_t n, int64_t R, int k,
                                int32_t* indices, void* ws, int mode, uint32_t* gflag, int G,
                                int pack, int64_t npacked, hipStream_t stream);
size_t scan_topk_workspace_bytes(int64_t groups, int G, int64_t n, int k);
hipError_t launch_scan_topk(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                            const uint8_t* depths, const float* q, int64_t groups, int G,
                            int64_t n, int k, float* scores, int32_t* indices, void* ws,
                            hipStream_t stream);
hipError_t launch_gather(const uint64_t* hplanes, const uint16_t* hscales, int64_t nb_store,
                         const uint8_t* depths, int64_t groups, int64_t n, uint64_t* planes,
                         uint16_t* scales, hipStream_t stream);
hipError_t launch_topk(const float* scores, int64_t rows, int64_t n, int k, int32_t* indices,
                       void* workspace, hipStream_t stream);
// fathom_topk with the library's fixed per-device scratch as its workspace
// (no allocation); hipErrorInvalidValue if the workspace would exceed it.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
hipError_t launch_topk_noalloc(const float* scores, int64_t rows, int64_t n, int k,
                               int32_t* indices, hipStream_t stream);

size_t klt_fit_workspace_bytes(int64_t groups, int64_t n);
hipError_t launch_klt_fit(const uint16_t* k, int64_t groups, int64_t n, float* mu, float* basis,
                          float* lambda, void* ws, hipStream_t stream);
hipError_t launch_klt_rotate_keys(const uint16_t* k, const float* mu, const float* basis,
                                  int64_t groups, int64_t n, uint16_t* out, hipStream_t stream);
hipError_t launch_klt_rotate_queries(const float* q, const float* basis, int64_t groups, int G,
                                     float* out, hipStream_t stream);

// Wave-wide helpers -------------------------------------------------------

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Make the wave's earlier LDS writes visible to its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace fathom
