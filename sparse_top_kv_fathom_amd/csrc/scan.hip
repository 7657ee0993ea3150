// fathom_scan on gfx950: approximate scores from the prefix bit planes.
//
// "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches",
// §3.2 (the first t planes are the t-bit mid-rise quantizer:
// khat = (c' + 0.5 - 2^(t-1)) * a / 2^(t-1), c' = c >> (4 - t)) and §3.3
// (channels with t = 0 are skipped; the plan is shared by the G heads of the
// group so the K bytes are read once for all of them); §7 prices the work at
// one multiply-add per active channel, token and head plus 1-2 integer ops
// per bit.
//
// Arithmetic.  Writing khat = a * (c' * 2^(1-t) + 2^-t - 1):
//   o_hb = fold_j fma(e_hj, a_bj, o),     e_hj = fl32(q_hj * (2^-t_j - 1))
//   S_hi = fold_j fma(w_hj, m_ij, S),     w_hj = q_hj * 2^(11-t_j),
//                                         m_ij = a_bj * c'_ij * 2^-10,
// folds over the active channels in ascending order, S starting at o.
//
// Mapping (wave64 = one 64-token block; lane i = token i = bit i of every
// plane word).  A plane word is loaded with a scalar load and used directly
// as the per-lane carry-in of v_addc_co_u32, so reading plane p costs one
// VALU instruction per block:  x <- 2x + bit_p.  Starting from 0x3C00 >> t,
// t steps leave x = 0x3C00 + c', the fp16 pattern of 1 + c' * 2^-10, and one
// v_fma_mix_f32 (fp16 a, fp16 x, -a) yields m = a * c' * 2^-10 exactly.
// Each head then costs one fp32 FMA.  Per block and active channel:
// t + 1 + G VALU instructions.  The per-block offsets o are computed first
// with lanes spread over (block, head) pairs and handed over through LDS, as
// are the per-channel coefficients w and the tile's block scales.
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kWaves = 4;        // waves per workgroup
constexpr int kNB = 8;           // blocks per wave tile (512 tokens)

// x <- 2x + (bit lane of mask): the plane word is the carry-in lane mask.
__device__ __forceinline__ uint32_t shift_in_plane(uint32_t x, uint64_t mask) {
  uint32_t r;
  asm("v_addc_co_u32_e64 %0, vcc, %1, %1, %2" : "=v"(r) : "v"(x), "s"(mask) : "vcc");
  return r;
}

__device__ __forceinline__ _Float16 as_half(uint32_t bits16) {
  return __builtin_bit_cast(_Float16, (uint16_t)bits16);
}

template <int G, int T>
__device__ __forceinline__ void accumulate_channel(const uint64_t* __restrict__ pj,
                                                   int64_t nb_store, int64_t last_off,
                                                   const uint32_t* __restrict__ s_a2,
                                                   const float (&w)[G], float (&acc)[kNB][G]) {
  constexpr uint32_t x0 = 0x3C00u >> T;
#pragma unroll
  for (int bl = 0; bl < kNB; ++bl) {
    // Blocks past the end of the scan range reread the last valid block; their
    // results are never stored.
    const int64_t off = bl < last_off ? bl : last_off;
    uint32_t x = x0;
#pragma unroll
    for (int p = 0; p < T; ++p) x = shift_in_plane(x, pj[p * nb_store + off]);
    const uint32_t a2 = s_a2[bl >> 1];
    const float a = (float)as_half((bl & 1) ? (a2 >> 16) : (a2 & 0xffffu));
    const float m = __builtin_fmaf(a, (float)as_half(x), -a);
#pragma unroll
    for (int h = 0; h < G; ++h) acc[bl][h] = __builtin_fmaf(w[h], m, acc[bl][h]);
  }
}

template <int G>
__global__ __launch_bounds__(kWaves * 64) void scan_kernel(
    const uint64_t* __restrict__ planes, const uint16_t* __restrict__ scales, int64_t nb_store,
    const uint8_t* __restrict__ depths, const float* __restrict__ q, int64_t nblk, int64_t n,
    float* __restrict__ scores) {
  static_assert(kNB * G <= 64, "one lane per (block, head) in the offset pass");
  __shared__ float s_w[kD][G];                    // q_hj * 2^(11 - t_j)
  __shared__ float s_e[kD][G];                    // fl32(q_hj * (2^-t_j - 1))
  __shared__ int s_act[kD];                       // active channels: j | t << 8, ascending
  __shared__ int s_nact;
  __shared__ float s_o[kWaves][kNB][G];           // per-block offsets of each wave tile
  __shared__ uint32_t s_a[kWaves][kD][kNB / 2];   // fp16 scales of the tile, per active slot

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int64_t grp = blockIdx.y;

  // Per-group tables (identical in every workgroup of the group).
  if (threadIdx.x < kD) {
    const int j = threadIdx.x;
    const int t = min((int)depths[grp * kD + j], kPlanes);  // depths above 4 read as 4
    const float sw = __builtin_ldexpf(1.0f, 11 - t);
    const float se = __builtin_ldexpf(1.0f, -t) - 1.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float qv = q[(grp * G + h) * kD + j];
      s_w[j][h] = qv * sw;
      s_e[j][h] = qv * se;
    }
  }
  if (wave == 0) {
    const int t0 = min((int)depths[grp * kD + lane], kPlanes);
    const int t1 = min((int)depths[grp * kD + 64 + lane], kPlanes);
    const uint64_t m0 = __ballot(t0 > 0);
    const uint64_t m1 = __ballot(t1 > 0);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int r0 = __popcll(m0 & below);
    const int r1 = __popcll(m0) + __popcll(m1 & below);
    if (t0 > 0) s_act[r0] = lane | (t0 << 8);
    if (t1 > 0) s_act[r1] = (lane + 64) | (t1 << 8);
    if (lane == 0) s_nact = __popcll(m0) + __popcll(m1);
  }
  __syncthreads();

  const int nact = s_nact;
  const int64_t blk0 = ((int64_t)blockIdx.x * kWaves + wave) * kNB;
  if (blk0 >= nblk) return;  // no further workgroup barriers below
  const int nvalid = (int)min<int64_t>(kNB, nblk - blk0);

  // Offsets o[b][h] and the tile's scales: lane = b * G + h.
  {
    const int bl = lane / G, h = lane % G;
    const bool on = lane < kNB * G;
    const int64_t blk = blk0 + min(bl, nvalid - 1);
    float o = 0.0f;
    for (int ai = 0; ai < nact; ++ai) {
      const int j = s_act[ai] & 0xff;
      const uint32_t a16 = on ? scales[(grp * kD + j) * nb_store + blk] : 0u;
      const float e = on ? s_e[j][h] : 0.0f;
      o = __builtin_fmaf(e, (float)as_half(a16), o);
      const uint32_t hi = __shfl_down(a16, G, 64);
      if (on && h == 0 && (bl & 1) == 0) s_a[wave][ai][bl >> 1] = a16 | (hi << 16);
    }
    if (on) s_o[wave][bl][h] = o;
  }
  wave_lds_sync();

  float acc[kNB][G];
#pragma unroll
  for (int bl = 0; bl < kNB; ++bl)
#pragma unroll
    for (int h = 0; h < G; ++h) acc[bl][h] = s_o[wave][bl][h];

  const int64_t last_off = nvalid - 1;
  for (int ai = 0; ai < nact; ++ai) {
    const int jt = __builtin_amdgcn_readfirstlane(s_act[ai]);
    const int j = jt & 0xff, t = jt >> 8;
    float w[G];
#pragma unroll
    for (int h = 0; h < G; ++h) w[h] = s_w[j][h];
    const uint64_t* pj = planes + (grp * kD + j) * (int64_t)kPlanes * nb_store + blk0;
    const uint32_t* a2 = &s_a[wave][ai][0];
    switch (t) {
      case 1: accumulate_channel<G, 1>(pj, nb_store, last_off, a2, w, acc); break;
      case 2: accumulate_channel<G, 2>(pj, nb_store, last_off, a2, w, acc); break;
      case 3: accumulate_channel<G, 3>(pj, nb_store, last_off, a2, w, acc); break;
      default: accumulate_channel<G, 4>(pj, nb_store, last_off, a2, w, acc); break;
    }
  }

#pragma unroll
  for (int bl = 0; bl < kNB; ++bl) {
    if (bl < nvalid) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        scores[(grp * G + h) * n + (blk0 + bl) * kBlock + lane] = acc[bl][h];
    }
  }
}

template <int G>
void launch_scan_g(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                   const uint8_t* depths, const float* q, int64_t groups, int64_t n,
                   float* scores, hipStream_t stream) {
  const int64_t nblk = n / kBlock;
  const int64_t per_wg = (int64_t)kWaves * kNB;
  dim3 grid((unsigned)((nblk + per_wg - 1) / per_wg), (unsigned)groups);
  hipLaunchKernelGGL(scan_kernel<G>, grid, dim3(kWaves * 64), 0, stream, planes, scales,
                     nb_store, depths, q, nblk, n, scores);
}

}  // namespace

hipError_t launch_scan(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                       const uint8_t* depths, const float* q, int64_t groups, int G, int64_t n,
                       float* scores, hipStream_t stream) {
  switch (G) {
    case 1: launch_scan_g<1>(planes, scales, nb_store, depths, q, groups, n, scores, stream); break;
    case 2: launch_scan_g<2>(planes, scales, nb_store, depths, q, groups, n, scores, stream); break;
    case 3: launch_scan_g<3>(planes, scales, nb_store, depths, q, groups, n, scores, stream); break;
    case 4: launch_scan_g<4>(planes, scales, nb_store, depths, q, groups, n, scores, stream); break;
    case 5: launch_scan_g<5>(planes, scales, nb_store, depths, q, groups, n, scores, stream); break;
    case 6: launch_scan_g<6>(planes, scales, nb_store, depths, q, groups, n, scores, stream); break;
    case 7: launch_scan_g<7>(planes, scales, nb_store, depths, q, groups, n, scores, stream); break;
    case 8: launch_scan_g<8>(planes, scales, nb_store, depths, q, groups, n, scores, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace fathom
