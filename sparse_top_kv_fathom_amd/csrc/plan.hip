// fathom_plan on gfx950: per query group importance and water-filling depths
// ("Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV
// Caches", §3.3 and Eq. 4): one wave64 per group runs plan_core::plan_group
// (plan_core.h).  Below it, the fixed-depth plans.
#include "fathom_internal.h"
#include "plan_core.h"

namespace fathom {
namespace {

template <int G>
__global__ __launch_bounds__(64) void plan_kernel(const float* __restrict__ q,
                                                  const float* __restrict__ var, int budget,
                                                  uint8_t* __restrict__ depths,
                                                  double* __restrict__ theta_out,
                                                  int32_t* __restrict__ bits_out) {
  plan_core::plan_group<G>(q, var, budget, depths, theta_out, bits_out, blockIdx.x);
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
