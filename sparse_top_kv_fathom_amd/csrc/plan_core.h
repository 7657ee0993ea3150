// The water-filling plan of one query group, run by one wave64: per query
// group importance and depths (fathom_plan, and the plan part of
// fathom_append_plan).
//
// "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches",
// §3.3 (Per-Query Read Depth) and Eq. 4, with the Appendix A walkthrough:
//   g_j = (sum_h q_hj^2) * Var_j,
//   t_j = clip(round(log4(g_j / theta)), 0, 4)      (halves rounded up)
//       = #{m in 1..4 : g_j >= 2^(2m-1) * theta},
//   theta = the smallest water line with sum_j t_j <= B, located by 30
//   geometric-midpoint bisection steps.
//
// Lane l owns channels l and l + 64.  The sum of depths at a trial theta is
// 8 ballots (4 thresholds x 2 channels) and their popcounts, so every step is
// a handful of instructions.  All comparisons are in fp64; 2^(2m-1) * theta
// is an exact scaling.
#pragma once

#include "fathom_internal.h"

namespace fathom {
namespace plan_core {

__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) v = fmax(v, __shfl_xor(v, s, 64));
  return v;
}

__device__ __forceinline__ double wave_min_f64(double v) {
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) v = fmin(v, __shfl_xor(v, s, 64));
  return v;
}

__device__ __forceinline__ int depth_of(double g, double theta) {
  // g > 0 is implied for theta > 0 by the first threshold.
  return (g >= 2.0 * theta) + (g >= 8.0 * theta) + (g >= 32.0 * theta) + (g >= 128.0 * theta);
}

__device__ __forceinline__ int sum_depths(double g0, double g1, double theta) {
  int s = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const double thr = theta * (double)(2 << (2 * m));  // 2, 8, 32, 128
    s += __popcll(__ballot(g0 >= thr)) + __popcll(__ballot(g1 >= thr));
  }
  return s;
}

template <int G>
__device__ __forceinline__ void plan_group(const float* __restrict__ q,
                                           const float* __restrict__ var, int budget,
                                           uint8_t* __restrict__ depths,
                                           double* __restrict__ theta_out,
                                           int32_t* __restrict__ bits_out, int64_t grp) {
  const int lane = lane_id();
  double gj[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int j = lane + 64 * c;
    double s = 0.0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const double x = (double)q[(grp * G + h) * kD + j];
      s = __dadd_rn(s, __dmul_rn(x, x));
    }
    gj[c] = __dmul_rn(s, (double)var[grp * kD + j]);
  }
  const bool p0 = gj[0] > 0.0, p1 = gj[1] > 0.0;
  const int npos = __popcll(__ballot(p0)) + __popcll(__ballot(p1));
  const double gmax = wave_max_f64(fmax(p0 ? gj[0] : 0.0, p1 ? gj[1] : 0.0));
  const double big = __builtin_huge_val();
  const double gmin = wave_min_f64(fmin(p0 ? gj[0] : big, p1 ? gj[1] : big));

  double theta;
  int t0, t1;
  if (npos == 0 || budget == 0) {
    theta = gmax;
    t0 = t1 = 0;
  } else if (budget >= 4 * npos) {
    theta = gmin / 256.0;
    t0 = p0 ? 4 : 0;
    t1 = p1 ? 4 : 0;
  } else {
    double lo = gmin / 256.0, hi = gmax;
    for (int step = 0; step < 30; ++step) {
      const double mid = __dsqrt_rn(__dmul_rn(lo, hi));
      if (sum_depths(gj[0], gj[1], mid) <= budget) hi = mid;
      else lo = mid;
    }
    theta = hi;
    t0 = depth_of(gj[0], hi);
    t1 = depth_of(gj[1], hi);
  }
  depths[grp * kD + lane] = (uint8_t)t0;
  depths[grp * kD + lane + 64] = (uint8_t)t1;
  if (theta_out != nullptr || bits_out != nullptr) {
    int used = t0 + t1;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) used += __shfl_xor(used, s, 64);
    if (lane == 0) {
      if (theta_out != nullptr) theta_out[grp] = theta;
      if (bits_out != nullptr) bits_out[grp] = used;
    }
  }
}

}  // namespace plan_core
}  // namespace fathom
