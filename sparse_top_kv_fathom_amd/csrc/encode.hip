// fathom_encode on gfx950: fp16 keys -> channel-major bit planes + fp16 scales.
//
// "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches",
// §3.2 (Bit-Plane K Cache): per 64-token block and channel, a = max |k|,
// s = a/8, code = clamp(floor(k/s) + 8, 0, 15); bit p of the 64 codes (p = 0
// the MSB) is one 64-bit plane word with token i in bit i.
//
// Mapping: one wave64 per 64-token block, lane i = token i, so each plane word
// is a single wave ballot.  The block max is a wave max of |k| taken on the
// fp16 bit patterns (positive fp16 patterns order like their values), two
// channels per 32-bit lane word.  A workgroup of 4 waves encodes 4 consecutive
// blocks; words and scales are staged in LDS and written as contiguous runs
// per (channel, plane).  Calls with few blocks use a column-split kernel
// instead (below).
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kWavesPerWg = 4;

// Max of two packed 16-bit lanes.
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Max of two packed 16-bit magnitudes across the wave, returned to every
// lane: DPP moves take the max within quads (lanes xor 1, xor 2), within rows
// of 16 (half mirror, mirror), then rows 0 and 2 into rows 1 and 3 (row
// broadcast of lane 15) and lanes 0-31 into rows 2 and 3 (broadcast of lane
// 31); lane 63 then holds the wave's max.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ uint32_t wave_max_u16x2(uint32_t v) {
  v = max_u16x2(v, dpp<0xB1, 0xf>(v));    // quad_perm [1, 0, 3, 2]
  v = max_u16x2(v, dpp<0x4E, 0xf>(v));    // quad_perm [2, 3, 0, 1]
  v = max_u16x2(v, dpp<0x141, 0xf>(v));   // row_half_mirror
  v = max_u16x2(v, dpp<0x140, 0xf>(v));   // row_mirror
  v = max_u16x2(v, dpp<0x142, 0xa>(v));   // row_bcast:15 into rows 1 and 3
  v = max_u16x2(v, dpp<0x143, 0xc>(v));   // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// 4-bit code of k (fp16 bits) in a block with max magnitude a (fp16 bits).
// floor(k / s) is formed from a reciprocal estimate and then corrected with
// exact products: m*s and (m+1)*s are exact in fp32 for |m| <= 9.
__device__ __forceinline__ uint32_t code_of(uint32_t kbits, uint32_t abits) {
  if (abits == 0) return 8u;
  const float a = f16_bits_to_float(abits);
  const float s = a * 0.125f;
  const float kf = f16_bits_to_float(kbits);
  float m = floorf(kf * (8.0f * __builtin_amdgcn_rcpf(a)));
  m = fminf(fmaxf(m, -9.0f), 9.0f);
  if (m * s > kf) m -= 1.0f;
  if ((m + 1.0f) * s <= kf) m += 1.0f;
  int c = (int)m + 8;
  c = c < 0 ? 0 : (c > 15 ? 15 : c);
  return (uint32_t)c;
}

__global__ __launch_bounds__(256) void encode_kernel(
    const uint16_t* __restrict__ k, int64_t n, int64_t nblk, int64_t nb_store,
    int64_t block_offset, uint64_t* __restrict__ planes, uint16_t* __restrict__ scales,
    uint32_t* __restrict__ flag) {
  __shared__ uint64_t s_words[kD][kPlanes][kWavesPerWg];
  __shared__ uint16_t s_scale[kD][kWavesPerWg];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t g = blockIdx.y;
  const int64_t blk0 = (int64_t)blockIdx.x * kWavesPerWg;
  const int64_t blk = blk0 + wave;
  const int nvalid = (int)min<int64_t>(kWavesPerWg, nblk - blk0);
  bool bad = false;

  if (wave < nvalid) {
    // Token row of this lane: 128 fp16 = 16 x 16 bytes.
    const uint4* row = reinterpret_cast<const uint4*>(k + ((g * n) + blk * kBlock + lane) * kD);
    for (int c = 0; c < kD / 8; ++c) {
      const uint4 v = row[c];
      const uint32_t w32[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t amax2 = wave_max_u16x2(w32[u] & 0x7fff7fffu);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int j = c * 8 + u * 2 + half;
          const uint32_t kb = (w32[u] >> (16 * half)) & 0xffffu;
          const uint32_t ab = (amax2 >> (16 * half)) & 0xffffu;
          bad |= ab >= 0x7c00u;  // Inf or NaN somewhere in the block
          const uint32_t code = code_of(kb, ab);
#pragma unroll
          for (int p = 0; p < kPlanes; ++p) {
            const uint64_t word = __ballot((code >> (3 - p)) & 1u);
            if (lane == p) s_words[j][p][wave] = word;
          }
          if (lane == 4) s_scale[j][wave] = (uint16_t)ab;
        }
      }
    }
  }
  if (flag != nullptr && bad && lane == 0) atomicOr(flag, 1u);
  __syncthreads();

  // Contiguous writes: for each (channel, plane), nvalid consecutive words.
  for (int idx = threadIdx.x; idx < kD * kPlanes * kWavesPerWg; idx += blockDim.x) {
    const int b = idx % kWavesPerWg;
    const int jp = idx / kWavesPerWg;
    const int j = jp / kPlanes, p = jp % kPlanes;
    if (b < nvalid)
      planes[((g * kD + j) * kPlanes + p) * nb_store + block_offset + blk0 + b] = s_words[j][p][b];
  }
  for (int idx = threadIdx.x; idx < kD * kWavesPerWg; idx += blockDim.x) {
    const int b = idx % kWavesPerWg;
    const int j = idx / kWavesPerWg;
    if (b < nvalid) scales[(g * kD + j) * nb_store + block_offset + blk0 + b] = s_scale[j][b];
  }
}

// Few blocks (the decode-time append of one block): the channels of a block
// are spread over 16 waves, one 16-byte column (8 channels) each, so the work
// of a block is not one wave's serial loop.  Grid: (blocks, groups, 4); the
// 4 waves of a workgroup take columns 4z .. 4z+3.  Words and scales are
// written directly (8 and 2 bytes per channel).
__global__ __launch_bounds__(256) void encode_cols_kernel(
    const uint16_t* __restrict__ k, int64_t n, int64_t nb_store, int64_t block_offset,
    uint64_t* __restrict__ planes, uint16_t* __restrict__ scales, uint32_t* __restrict__ flag) {
  const int lane = lane_id();
  const int col = blockIdx.z * kWavesPerWg + (threadIdx.x >> 6);   // 0..15
  const int64_t g = blockIdx.y;
  const int64_t blk = blockIdx.x;
  const uint4 v = *reinterpret_cast<const uint4*>(k + ((g * n) + blk * kBlock + lane) * kD + col * 8);
  const uint32_t w32[4] = {v.x, v.y, v.z, v.w};
  bool bad = false;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t amax2 = wave_max_u16x2(w32[u] & 0x7fff7fffu);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int64_t j = col * 8 + u * 2 + half;
      const uint32_t kb = (w32[u] >> (16 * half)) & 0xffffu;
      const uint32_t ab = (amax2 >> (16 * half)) & 0xffffu;
      bad |= ab >= 0x7c00u;
      const uint32_t code = code_of(kb, ab);
#pragma unroll
      for (int p = 0; p < kPlanes; ++p) {
        const uint64_t word = __ballot((code >> (3 - p)) & 1u);
        if (lane == p) planes[((g * kD + j) * kPlanes + p) * nb_store + block_offset + blk] = word;
      }
      if (lane == 4) scales[(g * kD + j) * nb_store + block_offset + blk] = (uint16_t)ab;
    }
  }
  if (flag != nullptr && bad && lane == 0) atomicOr(flag, 1u);
}

}  // namespace

// Below this many blocks per group the column-split kernel is used.
constexpr int64_t kColsKernelMaxBlocks = 64;

hipError_t launch_encode(const uint16_t* k, int64_t groups, int64_t n, int64_t nb_store,
                         int64_t block_offset, uint64_t* planes, uint16_t* scales,
                         uint32_t* nonfinite_flag, hipStream_t stream) {
  const int64_t nblk = n / kBlock;
  if (nblk <= kColsKernelMaxBlocks) {
    dim3 grid((unsigned)nblk, (unsigned)groups, kD / 8 / kWavesPerWg);
    hipLaunchKernelGGL(encode_cols_kernel, grid, dim3(64 * kWavesPerWg), 0, stream, k, n,
                       nb_store, block_offset, planes, scales, nonfinite_flag);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((nblk + kWavesPerWg - 1) / kWavesPerWg), (unsigned)groups);
  hipLaunchKernelGGL(encode_kernel, grid, dim3(64 * kWavesPerWg), 0, stream, k, n, nblk,
                     nb_store, block_offset, planes, scales, nonfinite_flag);
  return hipGetLastError();
}

}  // namespace fathom
