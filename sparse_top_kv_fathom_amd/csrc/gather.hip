// fathom_gather on gfx950: the runs a plan reads, from a host-resident store
// into the device store.
//
// "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches",
// §3.6: with the store channel-major, the first t_j planes of channel j are
// one contiguous run of t_j * n / 8 bytes (its scales a second run), so the
// bytes a plan needs move as a short list of long runs rather than as scattered
// words; §2 measures the host-resident regime and Fig. 10 the link rate of
// contiguous copies against word-by-word reads of mapped host memory.
//
// Mapping: the run list is implicit in the depths (device memory, so no host
// round trip): workgroup (segment, part, channel, group) copies one segment of
// 8192 blocks of plane `part` (part < 4, needed when part < t_j) or of the
// scale row (part 4, needed when t_j > 0) with 16-byte loads of the pinned
// host memory, eight in flight per thread, and 16-byte stores to HBM.
// Workgroups of runs the plan does not read return at once.
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kThreads = 256;
constexpr int kSegBlocks = 8192;          // blocks per workgroup segment
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void gather_kernel(const uint64_t* __restrict__ hplanes,
                                                          const uint16_t* __restrict__ hscales,
                                                          int64_t nb_store,
                                                          const uint8_t* __restrict__ depths,
                                                          int64_t nblk, uint64_t* __restrict__ planes,
                                                          uint16_t* __restrict__ scales) {
  const int64_t grp = blockIdx.z;
  const int j = blockIdx.y / 5, part = blockIdx.y % 5;
  const int t = min((int)depths[grp * kD + j], kPlanes);
  if (part < kPlanes ? part >= t : t == 0) return;
  const int64_t b0 = (int64_t)blockIdx.x * kSegBlocks;
  const int64_t b1 = min<int64_t>(nblk, b0 + kSegBlocks);
  if (b0 >= b1) return;
  // Byte range of the segment (rows are 16-byte aligned: nb_store % 8 == 0).
  const char* src;
  char* dst;
  int64_t bytes;
  if (part < kPlanes) {
    const int64_t row = ((grp * kD + j) * kPlanes + part) * nb_store;
    src = reinterpret_cast<const char*>(hplanes + row + b0);
    dst = reinterpret_cast<char*>(planes + row + b0);
    bytes = (b1 - b0) * 8;
  } else {
    const int64_t row = (grp * kD + j) * nb_store;
    src = reinterpret_cast<const char*>(hscales + row + b0);
    dst = reinterpret_cast<char*>(scales + row + b0);
    bytes = (b1 - b0) * 2;
  }
  const int64_t n16 = bytes / 16;
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  for (int64_t i0 = threadIdx.x; i0 < n16; i0 += kUnroll * kThreads) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * kThreads;
      if (i < n16) v[u] = s4[i];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + u * kThreads;
      if (i < n16) d4[i] = v[u];
    }
  }
  // A scale segment of a block count not a multiple of 8 ends in 2-byte words.
  for (int64_t i = n16 * 16 + threadIdx.x * 2; i < bytes; i += kThreads * 2)
    *reinterpret_cast<uint16_t*>(dst + i) = *reinterpret_cast<const uint16_t*>(src + i);
}

}  // namespace

hipError_t launch_gather(const uint64_t* hplanes, const uint16_t* hscales, int64_t nb_store,
                         const uint8_t* depths, int64_t groups, int64_t n, uint64_t* planes,
                         uint16_t* scales, hipStream_t stream) {
  const int64_t nblk = n / kBlock;
  const dim3 grid((unsigned)((nblk + kSegBlocks - 1) / kSegBlocks), 5 * kD, (unsigned)groups);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(kThreads), 0, stream, hplanes, hscales, nb_store,
                     depths, nblk, planes, scales);
  return hipGetLastError();
}

}  // namespace fathom
