// Workgroup selection primitives shared by the top-k kernels and by the
// scan's candidate cut: wave and workgroup prefix sums, the bin holding the
// need-th largest key of a histogram, and the two-digit radix cut.
#pragma once

#include "fathom_internal.h"
#include "topk_layout.h"

namespace fathom {
namespace topk {

// Inclusive prefix sum over the wave with DPP moves: shifts by 1, 2, 4 and 8
// lanes inside each row of 16 (lanes shifted in from outside the row read 0),
// then the last lane of row 0 added to row 1 and of row 2 to row 3
// (row_bcast:15), then lane 31 added to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  v = v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v = v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v = v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v = v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v = v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v = v + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Exclusive prefix over the NT threads of a workgroup; the total through
// `total`.
template <int NT>
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* s_tmp,
                                                        uint32_t& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_sum(v);
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t x = s_tmp[w];
    before += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

// Find, over bins held kPer per thread (highest bin last), the bin that
// holds the need-th largest key; thread-local h[] are the thread's bins.
// Writes (bin, need within the bin) to sel[] from the one thread that owns it.
template <int NT, int kPer>
__device__ __forceinline__ void pick_bin(const uint32_t (&h)[kPer], uint32_t need, uint32_t* s_tmp,
                                         uint32_t* sel) {
  uint32_t mine = 0;
#pragma unroll
  for (int b = 0; b < kPer; ++b) mine += h[b];
  uint32_t total;
  const uint32_t before = block_exclusive_sum<NT>(mine, s_tmp, total);
  const uint32_t above = total - before - mine;   // keys in higher bins
  if (above < need && need <= above + mine) {
    uint32_t acc = above;
#pragma unroll
    for (int b = kPer - 1; b >= 0; --b) {
      if (acc + h[b] >= need) {
        sel[0] = (uint32_t)(threadIdx.x * kPer + b);
        sel[1] = need - acc;
        break;
      }
      acc += h[b];
    }
  }
}

// The need-th largest of the keys of a workgroup of NT threads with its low
// 10 bits cleared: two radix digits of 11 bits over an LDS histogram (s_hist:
// kBins words, s_tmp: NT / 64, s_sel: 2).  visit(f) calls f(key) for each of
// the thread's keys, once per digit.  The result is at most 2^-13 of the
// score below that key, never above it.
template <int NT, class Visit>
__device__ __forceinline__ uint32_t radix_cut(Visit&& visit, uint32_t need, uint32_t* s_hist,
                                              uint32_t* s_tmp, uint32_t* s_sel) {
  uint32_t prefix = 0;
  for (int level = 0; level < 2; ++level) {
    const int shift = level == 0 ? 21 : 10;
    const int hi = shift + 11;   // bits at and above hi are fixed
    for (int i = threadIdx.x; i < kBins; i += NT) s_hist[i] = 0u;
    __syncthreads();
    visit([&](uint32_t key) {
      if (hi >= 32 || (key >> (hi & 31)) == (prefix >> (hi & 31)))
        atomicAdd(&s_hist[(key >> shift) & (kBins - 1)], 1u);
    });
    __syncthreads();
    constexpr int kPer = kBins / NT;
    uint32_t h[kPer];
#pragma unroll
    for (int b = 0; b < kPer; ++b) h[b] = s_hist[threadIdx.x * kPer + b];
    pick_bin<NT, kPer>(h, need, s_tmp, s_sel);
    __syncthreads();
    prefix |= s_sel[0] << shift;
    need = s_sel[1];
    __syncthreads();
  }
  return prefix;
}

}  // namespace topk
}  // namespace fathom
