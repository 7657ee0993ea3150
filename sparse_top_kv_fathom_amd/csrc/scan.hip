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
//   U_hi = fold_j fma(w_hj, m_ij, U),   U from +0,  w_hj = q_hj * 2^(11-t_j),
//                                                    m_ij = a_bj * c'_ij * 2^-10,
//   o_hb = fold_j fma(e_hj, a_bj, o),   o from +0,  e_hj = fl32(q_hj * (2^-t_j - 1)),
//   S_hi = fl32(U_hi + o_hb).
// Both folds visit the active channels by depth, deepest first, and by
// ascending channel index within a depth.  w and m are exact, so every fold
// step rounds once.
//
// Mapping.  A wave owns a tile of kNB consecutive 64-token blocks; lane i is
// token i of every block, i.e. bit i of every plane word.  The kNB plane words
// of one (channel, plane) are one scalar load, and a word is used directly as
// the per-lane carry-in of v_addc_co_u32, so plane p of a block costs one
// VALU instruction:  x <- 2x + bit_p.  Starting from 0x3C00 >> t, t steps
// leave x = 0x3C00 + c', the fp16 pattern of 1 + c' * 2^-10, and one
// v_fma_mix_f32 (fp16 scale a from an SGPR, fp16 x, -a) gives m exactly.
// Each head then costs one fp32 FMA.  The block offsets o are folded at the
// same time on kNB * G lanes (lane = block * G + head), one instruction per
// channel, and added in the epilogue.
//
// Latency.  Channels of one depth form a loop with a compile-time plane
// count; it is software-pipelined two deep (ping-pong register sets), so the
// scalar loads (planes, scales), LDS reads (w, e) and the vector load (the
// per-lane scale of the offset fold) of the next channel are in flight while
// the current one is computed.
//
// Grid.  A workgroup of kWaves waves covers kRounds * kWaves * kNB blocks of
// one group; workgroup ids are remapped so that consecutive tiles of a group
// run on the same XCD (workgroups are dealt to the 8 XCDs round-robin).  In
// the main kernel every tile is whole: a tile that would run past the last
// block is moved back to end on it and stores only its new blocks.  Stores
// with fewer than kNB blocks, or an odd block capacity (scale rows that are
// not 4-byte aligned), use the same kernel with per-block clamped loads.
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kWaves = 4;                    // waves per workgroup
constexpr int kNB = 4;                       // blocks per wave tile (256 tokens)
constexpr int kRounds = 4;                   // wave tiles per wave
constexpr int kWgBlocks = kWaves * kNB * kRounds;
constexpr int kXcds = 8;
// Byte offsets inside one group's plane array are 32-bit in the fast path.
constexpr int64_t kMaxFastBlocks = (int64_t(1) << 32) / (kD * kPlanes * 8) - 1;

// x <- 2x + (bit lane of mask): the plane word is the carry-in lane mask.
__device__ __forceinline__ uint32_t shift_in_plane(uint32_t x, uint64_t mask) {
  uint32_t r;
  asm("v_addc_co_u32_e64 %0, vcc, %1, %1, %2" : "=v"(r) : "v"(x), "s"(mask) : "vcc");
  return r;
}

__device__ __forceinline__ float half_lo(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

// Per-group tables shared by the waves of a workgroup, indexed by active
// slot (deepest channels first, ascending j within a depth).  Two padding
// slots let the pipeline read one slot past the end.
template <int G>
struct GroupTables {
  float w[kD + 2][G];        // q_hj * 2^(11 - t_j)
  float e[kD + 2][G];        // fl32(q_hj * (2^-t_j - 1))
  uint32_t poff[kD + 2];     // byte offset of the channel's plane rows in the group
  int count[kPlanes];        // number of active channels of depth 4, 3, 2, 1
};

// Everything one channel contributes to a wave tile.
template <int T, int G>
struct ChanLoad {
  uint64_t pw[T][kNB];   // plane words (wave-uniform)
  uint32_t a2[kNB / 2];  // block scales, two fp16 per dword (wave-uniform)
  float w[G];            // per-head weights (same in every lane)
  float e;               // offset coefficient of this lane's head
  uint32_t oa;           // scale of this lane's block (offset fold)
  uint32_t noff;         // plane offset of the following slot
};

struct TileCtx {
  const char* planes;       // the group's plane rows, advanced to the tile's first block
  const char* scales;       // the group's scale rows, advanced to the tile's first block
  uint32_t pstride;         // bytes between two planes of a channel (nb_store * 8)
  int last;                 // last valid block offset in the tile (clamped loads)
  uint32_t oa_off;          // this lane's byte offset in the offset fold (block * 2)
  int oh;                   // this lane's head in the offset fold
};

template <int T, int G, bool FULL>
__device__ __forceinline__ void load_chan(const TileCtx& c, const GroupTables<G>& tb, int slot,
                                          uint32_t off, ChanLoad<T, G>& L) {
  const char* rp = c.planes + off;
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int b = 0; b < kNB; ++b)
      L.pw[p][b] = *reinterpret_cast<const uint64_t*>(
          rp + p * c.pstride + (FULL ? b : min(b, c.last)) * 8);
  const char* sp = c.scales + (off >> 4);  // plane offset / 16 = scale-row offset
  if (FULL) {
    // Whole tiles of an even-capacity store: the kNB scales are aligned dwords.
#pragma unroll
    for (int i = 0; i < kNB / 2; ++i) L.a2[i] = reinterpret_cast<const uint32_t*>(sp)[i];
  } else {
    const uint16_t* hp = reinterpret_cast<const uint16_t*>(sp);
#pragma unroll
    for (int i = 0; i < kNB / 2; ++i)
      L.a2[i] = (uint32_t)hp[min(2 * i, c.last)] | ((uint32_t)hp[min(2 * i + 1, c.last)] << 16);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) L.w[h] = tb.w[slot][h];
  L.e = tb.e[slot][c.oh];
  L.oa = *reinterpret_cast<const uint16_t*>(sp + c.oa_off);
  L.noff = tb.poff[slot + 1];
}

template <int T, int G>
__device__ __forceinline__ void compute_chan(const ChanLoad<T, G>& L, float (&acc)[kNB][G],
                                             float& o) {
  constexpr uint32_t x0 = 0x3C00u >> T;
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    uint32_t x = x0;
#pragma unroll
    for (int p = 0; p < T; ++p) x = shift_in_plane(x, L.pw[p][b]);
    const uint32_t ab = (b & 1) ? (L.a2[b >> 1] >> 16) : L.a2[b >> 1];
    const float a = half_lo(ab);
    const float m = __builtin_fmaf(a, half_lo(x), -a);
#pragma unroll
    for (int h = 0; h < G; ++h) acc[b][h] = __builtin_fmaf(L.w[h], m, acc[b][h]);
  }
  o = __builtin_fmaf(L.e, half_lo(L.oa), o);
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// The channels of depth T: active slots [first, first + cnt).  Two register
// sets alternate; the loads of slot i + 1 are issued before slot i is
// computed.  The pipeline reads up to two slots past the range (padding or
// other active channels), which are never computed.
template <int T, int G, bool FULL>
__device__ __forceinline__ void depth_loop(const TileCtx& c, const GroupTables<G>& tb, int first,
                                           int cnt, float (&acc)[kNB][G], float& o) {
  if (cnt <= 0) return;
  ChanLoad<T, G> A, B;
  load_chan<T, G, FULL>(c, tb, first, uniform(tb.poff[first]), A);
  int i = 0;
  for (; i + 1 < cnt; i += 2) {
    load_chan<T, G, FULL>(c, tb, first + i + 1, uniform(A.noff), B);
    compute_chan<T, G>(A, acc, o);
    load_chan<T, G, FULL>(c, tb, first + i + 2, uniform(B.noff), A);
    compute_chan<T, G>(B, acc, o);
  }
  if (i < cnt) compute_chan<T, G>(A, acc, o);
}

// One wave tile of kNB blocks; blocks [store_from, store_to] (offsets in the
// tile) are stored.
template <int G, bool FULL>
__device__ __forceinline__ void scan_tile(const TileCtx& c, const GroupTables<G>& tb,
                                          int store_from, int store_to, int64_t n,
                                          float* __restrict__ out) {
  const int lane = lane_id();
  float acc[kNB][G];
#pragma unroll
  for (int b = 0; b < kNB; ++b)
#pragma unroll
    for (int h = 0; h < G; ++h) acc[b][h] = 0.0f;
  float o = 0.0f;

  const int c4 = tb.count[0], c3 = tb.count[1], c2 = tb.count[2], c1 = tb.count[3];
  depth_loop<4, G, FULL>(c, tb, 0, c4, acc, o);
  depth_loop<3, G, FULL>(c, tb, c4, c3, acc, o);
  depth_loop<2, G, FULL>(c, tb, c4 + c3, c2, acc, o);
  depth_loop<1, G, FULL>(c, tb, c4 + c3 + c2, c1, acc, o);

  // Epilogue: S = U + o (o of block b, head h sits in lane b * G + h).
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    if (b >= store_from && b <= store_to) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float obh = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, o), b * G + h));
        out[h * n + b * kBlock + lane] = acc[b][h] + obh;
      }
    }
  }
}

template <int G, bool FULL>
__global__ __launch_bounds__(kWaves * 64) void scan_kernel(
    const uint64_t* __restrict__ planes, const uint16_t* __restrict__ scales, int64_t nb_store,
    const uint8_t* __restrict__ depths, const float* __restrict__ q, int64_t nblk, int64_t n,
    int64_t wgs_per_group, float* __restrict__ scores) {
  static_assert(kNB * G <= 64, "one lane per (block, head) in the offset fold");
  __shared__ GroupTables<G> tb;

  // XCD-aware remap of the workgroup id (bijective on [0, gridDim.x)).
  const uint32_t nwg = gridDim.x;
  const uint32_t per_xcd = nwg / kXcds;
  uint32_t id = blockIdx.x;
  if (id < per_xcd * kXcds) id = (id % kXcds) * per_xcd + id / kXcds;
  const int64_t grp = id / wgs_per_group;
  const int64_t wg_in_grp = id % wgs_per_group;

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t pstride = (uint32_t)nb_store * 8u;

  if (wave < 2) {
    // Thread j < 128 owns channel j: its depth, its slot in the active list
    // (by depth 4, 3, 2, 1, ascending j within a depth) and its table row.
    const int j = threadIdx.x;
    const int t = min((int)depths[grp * kD + j], kPlanes);  // depths above 4 read as 4
    const int tlo = min((int)depths[grp * kD + lane], kPlanes);
    const int thi = min((int)depths[grp * kD + 64 + lane], kPlanes);
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int base = 0, slot = -1;
#pragma unroll
    for (int d = kPlanes; d >= 1; --d) {
      const uint64_t m0 = __ballot(tlo == d);
      const uint64_t m1 = __ballot(thi == d);
      const int cnt = __popcll(m0) + __popcll(m1);
      if (t == d) slot = base + (wave == 0 ? __popcll(m0 & below) : __popcll(m0) + __popcll(m1 & below));
      if (threadIdx.x == 0) tb.count[kPlanes - d] = cnt;
      base += cnt;
    }
    if (slot >= 0) {
      const float sw = __builtin_ldexpf(1.0f, 11 - t);
      const float se = __builtin_ldexpf(1.0f, -t) - 1.0f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float qv = q[(grp * G + h) * kD + j];
        tb.w[slot][h] = qv * sw;
        tb.e[slot][h] = qv * se;
      }
      tb.poff[slot] = (uint32_t)j * kPlanes * pstride;
    }
    // Padding slots (inactive tail of the list): channel 0, zero weights.
    const int nact_here = base;
    if (j >= nact_here && j < kD + 2) {
#pragma unroll
      for (int h = 0; h < G; ++h) tb.w[j][h] = tb.e[j][h] = 0.0f;
      tb.poff[j] = 0u;
    }
    if (j < 2) {
#pragma unroll
      for (int h = 0; h < G; ++h) tb.w[kD + j][h] = tb.e[kD + j][h] = 0.0f;
      tb.poff[kD + j] = 0u;
    }
  }
  __syncthreads();

  const bool olane = lane < kNB * G;
  const int ob = olane ? lane / G : 0;
  TileCtx c;
  c.pstride = pstride;
  c.oh = olane ? lane % G : 0;
  const char* planes_g = reinterpret_cast<const char*>(planes + grp * kD * (int64_t)kPlanes * nb_store);
  const char* scales_g = reinterpret_cast<const char*>(scales + grp * kD * nb_store);
  float* scores_g = scores + grp * G * n;

  for (int r = 0; r < kRounds; ++r) {
    const int64_t blk = wg_in_grp * kWgBlocks + ((int64_t)r * kWaves + wave) * kNB;
    if (blk >= nblk) break;
    if (FULL) {
      // Whole tile.  The last one is moved back to end on the last block, and
      // forward by one if that start is odd (scale dwords stay aligned; the
      // even capacity leaves room for the extra block, which is not stored).
      int64_t blk0 = min<int64_t>(blk, nblk - kNB);
      if (blk0 & 1) ++blk0;
      c.last = kNB - 1;
      c.oa_off = (uint32_t)ob * 2u;
      c.planes = planes_g + blk0 * 8;
      c.scales = scales_g + blk0 * 2;
      scan_tile<G, true>(c, tb, (int)(blk - blk0), (int)min<int64_t>(kNB - 1, nblk - 1 - blk0), n,
                         scores_g + blk0 * kBlock);
    } else {
      c.last = (int)min<int64_t>(kNB, nblk - blk) - 1;
      c.oa_off = (uint32_t)min(ob, c.last) * 2u;
      c.planes = planes_g + blk * 8;
      c.scales = scales_g + blk * 2;
      scan_tile<G, false>(c, tb, 0, c.last, n, scores_g + blk * kBlock);
    }
  }
}

template <int G>
void launch_scan_g(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                   const uint8_t* depths, const float* q, int64_t groups, int64_t n,
                   float* scores, hipStream_t stream) {
  const int64_t nblk = n / kBlock;
  const int64_t wgs_per_group = (nblk + kWgBlocks - 1) / kWgBlocks;
  const dim3 grid((unsigned)(wgs_per_group * groups));
  if (nblk >= kNB && nb_store % 2 == 0 && nb_store <= kMaxFastBlocks)
    hipLaunchKernelGGL((scan_kernel<G, true>), grid, dim3(kWaves * 64), 0, stream, planes,
                       scales, nb_store, depths, q, nblk, n, wgs_per_group, scores);
  else
    hipLaunchKernelGGL((scan_kernel<G, false>), grid, dim3(kWaves * 64), 0, stream, planes,
                       scales, nb_store, depths, q, nblk, n, wgs_per_group, scores);
}

}  // namespace

int64_t scan_max_workgroups(int64_t groups, int64_t n) {
  const int64_t nblk = n / kBlock;
  return groups * ((nblk + kWgBlocks - 1) / kWgBlocks);
}

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
