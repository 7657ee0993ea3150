// fathom_encode on gfx950: fp16 keys -> channel-major bit planes + fp16 scales.
//
// "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches",
// §3.2 (Bit-Plane K Cache): per 64-token block and channel, a = max |k|,
// s = a/8, code = clamp(floor(k/s) + 8, 0, 15); bit p of the 64 codes (p = 0
// the MSB) is one 64-bit plane word with token i in bit i.
//
// The code is found bit by bit, MSB first, by comparing k with a threshold
// that is an integer multiple of s (exact in fp32), so a channel and token
// cost four compares, three selects and two adds (code_bits below).
//
// Whole stores: one wave64 per 64-token block, lane l owns channels 2l and
// 2l + 1 (one 32-bit word of every token row: the wave's loads of one token
// are 256 contiguous bytes), holds the block's 64 words in registers, takes
// the block max of both channels with packed 16-bit maxima of the fp16
// magnitude bits (positive fp16 patterns order like their values), then
// walks the tokens from 63 down to 0 and shifts each code bit into its
// plane word through the carry-in of one add, so the lane ends with its two
// channels' 8 plane words.  A workgroup of 8 waves encodes 8 consecutive
// blocks; words and scales are staged in LDS and written as 64-byte runs per
// (channel, plane).  Calls with few blocks use a column-split kernel instead
// (below), which spreads a block's channels over waves with lane = token.
#include "fathom_internal.h"
#include "plan_core.h"

namespace fathom {
namespace {

constexpr int kWavesPerWg = 4;    // column-split kernel
constexpr int kStoreWaves = 8;    // whole-store kernel: blocks per workgroup

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

// The 4 plane words of one channel of a block, lane i holding token i's value
// kf (an fp16 value in fp32) and every lane the block's max magnitude `ab`
// (fp16 bits).  The code c = clamp(floor(k/s) + 8, 0, 15), s = a/8, is the
// largest c in [0, 15] with (c - 8) s <= k: taken MSB first, bit p is 1 when
// k >= (c_p + 2^(3-p) - 8) s, c_p the bits above it.  Every threshold is
// +-4s, then +-2s, then +-s added: an integer multiple of s below 8s in
// magnitude, exact in fp32 (s has an fp16 mantissa; a/8 is exact), so each
// compare is exact and its lane mask is plane word p.  a = 0 (all-zero block)
// gives code 8: plane 0 all ones (every k is +-0), the others 0.
struct Planes4 {
  uint64_t w[kPlanes];
};

__device__ __forceinline__ Planes4 code_planes(float kf, uint32_t ab) {
  const float a = f16_bits_to_float(ab);
  const float s4 = a * 0.5f, s2 = a * 0.25f, s1 = a * 0.125f;
  const bool b0 = kf >= 0.0f;
  const float t1 = b0 ? s4 : -s4;
  const bool b1 = kf >= t1;
  const float t2 = t1 + (b1 ? s2 : -s2);
  const bool b2 = kf >= t2;
  const float t3 = t2 + (b2 ? s1 : -s1);
  const bool b3 = kf >= t3;
  const uint64_t nz = ab != 0u ? ~0ull : 0ull;   // uniform
  Planes4 r;
  r.w[0] = __ballot(b0);
  r.w[1] = __ballot(b1) & nz;
  r.w[2] = __ballot(b2) & nz;
  r.w[3] = __ballot(b3) & nz;
  return r;
}

// x <- 2x + (this lane's bit of `mask`): the mask is the carry-in of one add;
// the carry-out (always 0: 32 steps from 0 stay below 2^32) goes to a scratch
// scalar pair.
__device__ __forceinline__ uint32_t shift_in(uint32_t x, uint64_t mask) {
  uint32_t r;
  uint64_t co;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=&s"(co) : "v"(x), "s"(mask));
  return r;
}

// One token of one channel in the whole-store kernel: the four code bits of
// kf (see code_planes) shifted into the lane's plane-word halves w[0..3].
__device__ __forceinline__ void code_bits(float kf, float s4, float s2, float s1,
                                          uint32_t (&w)[kPlanes]) {
  const bool b0 = kf >= 0.0f;
  w[0] = shift_in(w[0], __ballot(b0));
  const float t1 = b0 ? s4 : -s4;
  const bool b1 = kf >= t1;
  w[1] = shift_in(w[1], __ballot(b1));
  const float t2 = t1 + (b1 ? s2 : -s2);
  const bool b2 = kf >= t2;
  w[2] = shift_in(w[2], __ballot(b2));
  const float t3 = t2 + (b2 ? s1 : -s1);
  w[3] = shift_in(w[3], __ballot(kf >= t3));
}

// Lane LANE of `old` set to the wave-uniform `val` (the lane is an inline
// constant, so no lane-select hazard).
template <int LANE>
__device__ __forceinline__ uint32_t write_lane(uint32_t old, uint32_t val) {
  static_assert(LANE >= 0 && LANE < 64, "a lane of the wave");
  asm("v_writelane_b32 %0, %1, %2" : "+v"(old) : "s"(val), "i"(LANE));
  return old;
}

// The plane words and scales of 8 channels of a block (one 16-byte column of
// the token rows: lane i holds token i's 8 values): word dword L % 2 of
// (channel L / 8, plane (L / 2) % 4) in lane L of `words`, the scale of
// channel L in lane L < 8 of `sc`.
template <int JJ>
__device__ __forceinline__ void encode_chan(uint32_t kb, uint32_t ab, uint32_t& words,
                                            uint32_t& sc, bool& bad) {
  bad |= ab >= 0x7c00u;   // Inf or NaN somewhere in the block
  const Planes4 P = code_planes(f16_bits_to_float(kb), ab);
  words = write_lane<JJ * 8 + 0>(words, (uint32_t)P.w[0]);
  words = write_lane<JJ * 8 + 1>(words, (uint32_t)(P.w[0] >> 32));
  words = write_lane<JJ * 8 + 2>(words, (uint32_t)P.w[1]);
  words = write_lane<JJ * 8 + 3>(words, (uint32_t)(P.w[1] >> 32));
  words = write_lane<JJ * 8 + 4>(words, (uint32_t)P.w[2]);
  words = write_lane<JJ * 8 + 5>(words, (uint32_t)(P.w[2] >> 32));
  words = write_lane<JJ * 8 + 6>(words, (uint32_t)P.w[3]);
  words = write_lane<JJ * 8 + 7>(words, (uint32_t)(P.w[3] >> 32));
  sc = write_lane<JJ>(sc, ab);
}

// Channels 2U and 2U + 1 of the column (the two halves of lane word w).
template <int U>
__device__ __forceinline__ void encode_pair(uint32_t w, uint32_t& words, uint32_t& sc, bool& bad) {
  const uint32_t amax2 = wave_max_u16x2(w & 0x7fff7fffu);
  encode_chan<2 * U>(w & 0xffffu, amax2 & 0xffffu, words, sc, bad);
  encode_chan<2 * U + 1>(w >> 16, amax2 >> 16, words, sc, bad);
}

__device__ __forceinline__ void encode_column(const uint4 v, uint32_t& words, uint32_t& sc,
                                              bool& bad) {
  const uint32_t w32[4] = {v.x, v.y, v.z, v.w};
  encode_pair<0>(w32[0], words, sc, bad);
  encode_pair<1>(w32[1], words, sc, bad);
  encode_pair<2>(w32[2], words, sc, bad);
  encode_pair<3>(w32[3], words, sc, bad);
}

__global__ __launch_bounds__(kStoreWaves * 64) void encode_kernel(
    const uint16_t* __restrict__ k, int64_t n, int64_t nblk, int64_t nb_store,
    int64_t block_offset, uint64_t* __restrict__ planes, uint16_t* __restrict__ scales,
    uint32_t* __restrict__ flag) {
  __shared__ uint64_t s_words[kD][kPlanes][kStoreWaves];
  __shared__ uint16_t s_scale[kD][kStoreWaves];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t g = blockIdx.y;
  const int64_t blk0 = (int64_t)blockIdx.x * kStoreWaves;
  const int64_t blk = blk0 + wave;
  const int nvalid = (int)min<int64_t>(kStoreWaves, nblk - blk0);
  bool bad = false;

  if (wave < nvalid) {
    // Word l (channels 2l, 2l + 1) of the block's 64 token rows.
    const uint32_t* src = reinterpret_cast<const uint32_t*>(k + (g * n + blk * kBlock) * kD) + lane;
    uint32_t v[kBlock];
#pragma unroll
    for (int t = 0; t < kBlock; ++t) v[t] = src[t * (kD / 2)];
    uint32_t amax2 = 0u;
#pragma unroll
    for (int t = 0; t < kBlock; ++t) amax2 = max_u16x2(amax2, v[t] & 0x7fff7fffu);
    bad = (amax2 & 0xffffu) >= 0x7c00u || (amax2 >> 16) >= 0x7c00u;   // Inf or NaN
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t ab = (amax2 >> (16 * h)) & 0xffffu;
      const float a = f16_bits_to_float(ab);
      const float s4 = a * 0.5f, s2 = a * 0.25f, s1 = a * 0.125f;
      uint32_t hi[kPlanes] = {0u, 0u, 0u, 0u}, lo[kPlanes] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int t = kBlock - 1; t >= 32; --t)
        code_bits(f16_bits_to_float((v[t] >> (16 * h)) & 0xffffu), s4, s2, s1, hi);
#pragma unroll
      for (int t = 31; t >= 0; --t)
        code_bits(f16_bits_to_float((v[t] >> (16 * h)) & 0xffffu), s4, s2, s1, lo);
      // a = 0 (all-zero block): code 8 in every token.
      const int c = 2 * lane + h;
#pragma unroll
      for (int p = 0; p < kPlanes; ++p) {
        uint64_t w = ((uint64_t)hi[p] << 32) | lo[p];
        if (ab == 0u) w = p == 0 ? ~0ull : 0ull;
        s_words[c][p][wave] = w;
      }
      s_scale[c][wave] = (uint16_t)ab;
    }
  }
  if (flag != nullptr && __ballot(bad) != 0ull && lane == 0) atomicOr(flag, 1u);
  __syncthreads();

  // Contiguous writes: for each (channel, plane), nvalid consecutive words.
  for (int idx = threadIdx.x; idx < kD * kPlanes * kStoreWaves; idx += blockDim.x) {
    const int b = idx % kStoreWaves;
    const int jp = idx / kStoreWaves;
    const int j = jp / kPlanes, p = jp % kPlanes;
    if (b < nvalid)
      planes[((g * kD + j) * kPlanes + p) * nb_store + block_offset + blk0 + b] = s_words[j][p][b];
  }
  for (int idx = threadIdx.x; idx < kD * kStoreWaves; idx += blockDim.x) {
    const int b = idx % kStoreWaves;
    const int j = idx / kStoreWaves;
    if (b < nvalid) scales[(g * kD + j) * nb_store + block_offset + blk0 + b] = s_scale[j][b];
  }
}

// Few blocks (the decode-time append of one block): the channels of a block
// are spread over 16 waves, one 16-byte column (8 channels) each, so the work
// of a block is not one wave's serial loop.  Grid: (blocks, groups, 4); the
// 4 waves of a workgroup take columns 4z .. 4z+3.  Words and scales are
// written directly, one 32-bit half of a word per lane.
__device__ __forceinline__ void encode_cols_block(
    const uint16_t* __restrict__ k, int64_t n, int64_t nb_store, int64_t block_offset,
    uint64_t* __restrict__ planes, uint16_t* __restrict__ scales, uint32_t* __restrict__ flag,
    int64_t g, int64_t blk, int z) {
  const int lane = lane_id();
  const int col = z * kWavesPerWg + (threadIdx.x >> 6);   // 0..15
  const uint4 v = *reinterpret_cast<const uint4*>(k + ((g * n) + blk * kBlock + lane) * kD + col * 8);
  bool bad = false;
  uint32_t words = 0u, sc = 0u;
  encode_column(v, words, sc, bad);
  const int64_t slot = block_offset + blk;
  const int64_t j = col * 8 + lane / 8;
  reinterpret_cast<uint32_t*>(planes + ((g * kD + j) * kPlanes + (lane / 2) % kPlanes) * nb_store +
                              slot)[lane % 2] = words;
  if (lane < 8) scales[(g * kD + col * 8 + lane) * nb_store + slot] = (uint16_t)sc;
  if (flag != nullptr && bad && lane == 0) atomicOr(flag, 1u);
}

__global__ __launch_bounds__(256) void encode_cols_kernel(
    const uint16_t* __restrict__ k, int64_t n, int64_t nb_store, int64_t block_offset,
    uint64_t* __restrict__ planes, uint16_t* __restrict__ scales, uint32_t* __restrict__ flag) {
  encode_cols_block(k, n, nb_store, block_offset, planes, scales, flag, blockIdx.y, blockIdx.x,
                    blockIdx.z);
}

// fathom_append_plan: a decode step's append and plan in one launch (they
// read and write disjoint data).  Workgroups [0, groups) plan one group each
// (wave 0: plan_core::plan_group; they come first, as the plan is the longer
// chain); the others encode the appended blocks as encode_cols_kernel does,
// workgroup groups + (g * nblk + blk) * 4 + z taking block blk of group g,
// columns 4z .. 4z+3.
template <int G>
__global__ __launch_bounds__(256) void append_plan_kernel(
    const uint16_t* __restrict__ k, int64_t n, int64_t nb_store, int64_t block_offset,
    uint64_t* __restrict__ planes, uint16_t* __restrict__ scales, uint32_t* __restrict__ flag,
    int64_t groups, const float* __restrict__ q, const float* __restrict__ var, int budget,
    uint8_t* __restrict__ depths, double* __restrict__ theta, int32_t* __restrict__ bits) {
  const int64_t id = blockIdx.x;
  if (id < groups) {
    if (threadIdx.x < 64) plan_core::plan_group<G>(q, var, budget, depths, theta, bits, id);
    return;
  }
  const int64_t nblk = n / kBlock;
  const int64_t e = id - groups;
  const int z = (int)(e % (kD / 8 / kWavesPerWg));
  const int64_t gb = e / (kD / 8 / kWavesPerWg);
  encode_cols_block(k, n, nb_store, block_offset, planes, scales, flag, gb / nblk, gb % nblk, z);
}

template <int G>
void launch_append_plan_g(const uint16_t* k, int64_t groups, int64_t n, int64_t nb_store,
                          int64_t block_offset, uint64_t* planes, uint16_t* scales,
                          uint32_t* flag, const float* q, const float* var, int budget,
                          uint8_t* depths, double* theta, int32_t* bits, hipStream_t stream) {
  const int64_t wgs = groups + groups * (n / kBlock) * (kD / 8 / kWavesPerWg);
  hipLaunchKernelGGL(append_plan_kernel<G>, dim3((unsigned)wgs), dim3(64 * kWavesPerWg), 0,
                     stream, k, n, nb_store, block_offset, planes, scales, flag, groups, q, var,
                     budget, depths, theta, bits);
}

}  // namespace

// Below this many blocks per group the column-split kernel is used.
constexpr int64_t kColsKernelMaxBlocks = 64;

hipError_t launch_append_plan(const uint16_t* k, int64_t groups, int64_t n, int64_t nb_store,
                              int64_t block_offset, uint64_t* planes, uint16_t* scales,
                              uint32_t* nonfinite_flag, const float* q, const float* var, int G,
                              int budget_bits, uint8_t* depths, double* theta,
                              int32_t* bits_used, hipStream_t stream) {
  if (n / kBlock > kColsKernelMaxBlocks) {   // not an append: the two launches
    hipError_t e = launch_encode(k, groups, n, nb_store, block_offset, planes, scales,
                                 nonfinite_flag, stream);
    if (e != hipSuccess) return e;
    return launch_plan(q, var, groups, G, budget_bits, depths, theta, bits_used, stream);
  }
  switch (G) {
#define FATHOM_APPEND_PLAN_CASE(GG)                                                          \
  case GG:                                                                                  \
    launch_append_plan_g<GG>(k, groups, n, nb_store, block_offset, planes, scales,          \
                             nonfinite_flag, q, var, budget_bits, depths, theta, bits_used, \
                             stream);                                                       \
    break;
    FATHOM_APPEND_PLAN_CASE(1)
    FATHOM_APPEND_PLAN_CASE(2)
    FATHOM_APPEND_PLAN_CASE(3)
    FATHOM_APPEND_PLAN_CASE(4)
    FATHOM_APPEND_PLAN_CASE(5)
    FATHOM_APPEND_PLAN_CASE(6)
    FATHOM_APPEND_PLAN_CASE(7)
    FATHOM_APPEND_PLAN_CASE(8)
#undef FATHOM_APPEND_PLAN_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

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
  dim3 grid((unsigned)((nblk + kStoreWaves - 1) / kStoreWaves), (unsigned)groups);
  hipLaunchKernelGGL(encode_kernel, grid, dim3(64 * kStoreWaves), 0, stream, k, n, nblk,
                     nb_store, block_offset, planes, scales, nonfinite_flag);
  return hipGetLastError();
}

}  // namespace fathom
