// fathom_plan on gfx950: per query group importance and water-filling depths.
//
// "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches",
// §3.3 (Per-Query Read Depth) and Eq. 4, with the Appendix A walkthrough:
//   g_j = (sum_h q_hj^2) * Var_j,
//   t_j = clip(round(log4(g_j / theta)), 0, 4)      (halves rounded up)
//       = #{m in 1..4 : g_j >= 2^(2m-1) * theta},
//   theta = the smallest water line with sum_j t_j <= B, located by 30
//   geometric-midpoint bisection steps.
//
// Mapping: one wave64 per group; lane l owns channels l and l + 64.  The sum
// of depths at a trial theta is 8 ballots (4 thresholds x 2 channels) and
// their popcounts, so every step is a handful of instructions.  All
// comparisons are in fp64; 2^(2m-1) * theta is an exact scaling.
#include "fathom_internal.h"

namespace fathom {
namespace {

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
__global__ __launch_bounds__(64) void plan_kernel(const float* __restrict__ q,
                                                  const float* __restrict__ var, int budget,
                                                  uint8_t* __restrict__ depths,
                                                  double* __restrict__ theta_out,
                                                  int32_t* __restrict__ bits_out) {
  const int64_t grp = blockIdx.x;
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

template <int G>
void launch_plan_g(const float* q, const float* var, int64_t groups, int budget,
                   uint8_t* depths, double* theta, int32_t* bits, hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel<G>, dim3((unsigned)groups), dim3(64), 0, stream, q, var,
                     budget, depths, theta, bits);
}

// Fixed-depth plans (the comparison points of the pages' evaluation, read
// through the same store and scan): every channel at one depth (the 2-bit
// thumbnail, the full 4-bit scan), or depth 4 on the r channels with the
// largest statistic and 0 elsewhere — SparQ's sum over the query heads of
// |q_hj| (fp64, heads in order), or a caller's per-channel statistic (a
// fixed set chosen offline, as Double Sparsity's).  Ties go to the lower
// channel index.  One wave per group; lane l owns channels l and l + 64.
template <int G>
__global__ __launch_bounds__(64) void plan_fixed_kernel(const float* __restrict__ q,
                                                        const float* __restrict__ stat, int mode,
                                                        int param, uint8_t* __restrict__ depths) {
  __shared__ double s_stat[kD];
  const int64_t grp = blockIdx.x;
  const int lane = lane_id();
  if (mode == FATHOM_PLAN_UNIFORM) {
    depths[grp * kD + lane] = (uint8_t)param;
    depths[grp * kD + lane + 64] = (uint8_t)param;
    return;
  }
  double v[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int j = lane + 64 * c;
    if (mode == FATHOM_PLAN_SPARQ) {
      double s = 0.0;
#pragma unroll
      for (int h = 0; h < G; ++h) s = __dadd_rn(s, fabs((double)q[(grp * G + h) * kD + j]));
      v[c] = s;
    } else {
      v[c] = (double)stat[grp * kD + j];
    }
    s_stat[j] = v[c];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int j = lane + 64 * c;
    int rank = 0;   // channels ahead of j: larger statistic, or equal with a lower index
    for (int i = 0; i < kD; ++i) {
      const double o = s_stat[i];
      rank += (o > v[c] || (o == v[c] && i < j)) ? 1 : 0;
    }
    depths[grp * kD + j] = rank < param ? (uint8_t)kPlanes : (uint8_t)0;
  }
}

template <int G>
void launch_plan_fixed_g(const float* q, const float* stat, int64_t groups, int mode, int param,
                         uint8_t* depths, hipStream_t stream) {
  hipLaunchKernelGGL(plan_fixed_kernel<G>, dim3((unsigned)groups), dim3(64), 0, stream, q, stat,
                     mode, param, depths);
}

}  // namespace

hipError_t launch_plan(const float* q, const float* var, int64_t groups, int G,
                       int budget_bits, uint8_t* depths, double* theta, int32_t* bits_used,
                       hipStream_t stream) {
  switch (G) {
    case 1: launch_plan_g<1>(q, var, groups, budget_bits, depths, theta, bits_used, stream); break;
    case 2: launch_plan_g<2>(q, var, groups, budget_bits, depths, theta, bits_used, stream); break;
    case 3: launch_plan_g<3>(q, var, groups, budget_bits, depths, theta, bits_used, stream); break;
    case 4: launch_plan_g<4>(q, var, groups, budget_bits, depths, theta, bits_used, stream); break;
    case 5: launch_plan_g<5>(q, var, groups, budget_bits, depths, theta, bits_used, stream); break;
    case 6: launch_plan_g<6>(q, var, groups, budget_bits, depths, theta, bits_used, stream); break;
    case 7: launch_plan_g<7>(q, var, groups, budget_bits, depths, theta, bits_used, stream); break;
    case 8: launch_plan_g<8>(q, var, groups, budget_bits, depths, theta, bits_used, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_plan_fixed(const float* q, const float* stat, int64_t groups, int G, int mode,
                             int param, uint8_t* depths, hipStream_t stream) {
  switch (G) {
    case 1: launch_plan_fixed_g<1>(q, stat, groups, mode, param, depths, stream); break;
    case 2: launch_plan_fixed_g<2>(q, stat, groups, mode, param, depths, stream); break;
    case 3: launch_plan_fixed_g<3>(q, stat, groups, mode, param, depths, stream); break;
    case 4: launch_plan_fixed_g<4>(q, stat, groups, mode, param, depths, stream); break;
    case 5: launch_plan_fixed_g<5>(q, stat, groups, mode, param, depths, stream); break;
    case 6: launch_plan_fixed_g<6>(q, stat, groups, mode, param, depths, stream); break;
    case 7: launch_plan_fixed_g<7>(q, stat, groups, mode, param, depths, stream); break;
    case 8: launch_plan_fixed_g<8>(q, stat, groups, mode, param, depths, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fathom
