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
// v_fma_mix_f32 (fp16 scale a, fp16 x, -a) gives m exactly.  Each head then
// costs one fp32 FMA.  The block offsets o are folded at the same time on
// kNB * G lanes (lane = block * G + head), one instruction per channel, and
// added in the epilogue.
//
// Latency.  A workgroup walks "rounds" of kWaves * kNB blocks.  While round r
// is computed, the workgroup touches every plane line of round r + 1 with
// vector loads (so the scalar loads of round r + 1 find them in L2) and
// stages the block scales of round r + 1 in LDS.  Inside a round, channels of
// one depth form a loop with a compile-time plane count, software-pipelined
// two deep (ping-pong register sets): the scalar plane loads and the LDS reads
// of the next channel are in flight while the current one is computed.
//
// Grid.  Main kernel: whole rounds only; workgroup ids are remapped so that
// consecutive rounds of a group run on the same XCD (workgroups are dealt to
// the 8 XCDs round-robin).  The blocks after the last whole round (fewer
// than kWaves * kNB per group) go to a small tail kernel with per-block
// clamped loads, which also serves stores too large for 32-bit offsets.
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kWaves = 4;                    // waves per workgroup
constexpr int kNB = 4;                       // blocks per wave tile (256 tokens)
constexpr int kRoundBlocks = kWaves * kNB;   // blocks per workgroup round
constexpr int kRounds = 4;                   // rounds per workgroup (main kernel)
constexpr int kXcds = 8;
constexpr int kSlots = kD + 2;               // active slots + two padding slots
// Byte offsets inside one group's plane array are 32-bit in the main kernel.
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

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// Per-group tables shared by the waves of a workgroup, indexed by active
// slot (deepest channels first, ascending j within a depth).  The padding
// slots (zero weights, channel 0) let the pipeline read past the end.
template <int G>
struct GroupTables {
  float w[kSlots][G];           // q_hj * 2^(11 - t_j)
  float e[kSlots][G];           // fl32(q_hj * (2^-t_j - 1))
  uint32_t poff[kSlots];        // j * 4 * pstride: the channel's plane rows in the group
  uint32_t prow[kD * kPlanes];  // poff + p * pstride of every active plane row
  int count[kPlanes];           // number of active channels of depth 4, 3, 2, 1
  int nact, nrows;
};

// Build the tables of group `grp` with the 2 x 64 threads of waves 0 and 1
// (thread j owns channel j); the caller synchronises afterwards.
template <int G>
__device__ __forceinline__ void build_tables(GroupTables<G>& tb, const uint8_t* __restrict__ depths,
                                             const float* __restrict__ q, int64_t grp,
                                             uint32_t pstride) {
  const int tid = threadIdx.x;
  if (tid >= 2 * 64) return;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int j = tid;
  const int t = min((int)depths[grp * kD + j], kPlanes);  // depths above 4 read as 4
  const int tlo = min((int)depths[grp * kD + lane], kPlanes);
  const int thi = min((int)depths[grp * kD + 64 + lane], kPlanes);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base = 0, rows = 0, slot = -1, row0 = 0;
#pragma unroll
  for (int d = kPlanes; d >= 1; --d) {
    const uint64_t m0 = __ballot(tlo == d);
    const uint64_t m1 = __ballot(thi == d);
    const int cnt = __popcll(m0) + __popcll(m1);
    if (t == d) {
      const int rank = wave == 0 ? __popcll(m0 & below) : __popcll(m0) + __popcll(m1 & below);
      slot = base + rank;
      row0 = rows + rank * d;
    }
    if (tid == 0) tb.count[kPlanes - d] = cnt;
    base += cnt;
    rows += cnt * d;
  }
  if (tid == 0) {
    tb.nact = base;
    tb.nrows = rows;
  }
  const uint32_t poff = (uint32_t)j * kPlanes * pstride;
  if (slot >= 0) {
    const float sw = __builtin_ldexpf(1.0f, 11 - t);
    const float se = __builtin_ldexpf(1.0f, -t) - 1.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float qv = q[(grp * G + h) * kD + j];
      tb.w[slot][h] = qv * sw;
      tb.e[slot][h] = qv * se;
    }
    tb.poff[slot] = poff;
    for (int p = 0; p < t; ++p) tb.prow[row0 + p] = poff + (uint32_t)p * pstride;
  }
  // Padding slots [nact, kSlots): channel 0 with zero weights.
  for (int s = base + j; s < kSlots; s += 2 * 64) {
#pragma unroll
    for (int h = 0; h < G; ++h) tb.w[s][h] = tb.e[s][h] = 0.0f;
    tb.poff[s] = 0u;
  }
}

// Everything one channel contributes to a wave tile.
template <int T, int G>
struct ChanLoad {
  uint64_t pw[T][kNB];   // plane words (wave-uniform)
  uint32_t a2[kNB / 2];  // block scales, two fp16 per dword (same in every lane)
  float w[G];            // per-head weights (same in every lane)
  float e;               // offset coefficient of this lane's head
  uint32_t oa;           // scale of this lane's block (offset fold)
  uint32_t noff;         // plane offset of the following slot
};

// Channel of depth T for the wave tile.  `issue_next` runs right after the
// first instruction that reads this channel's loaded registers: scalar loads
// return out of order, so the only usable wait is "all outstanding", and it
// must land before the next channel's loads are issued, not after.  The
// scheduling barriers keep the compiler from moving loads across that point.
template <int T, int G, class F>
__device__ __forceinline__ void compute_chan(const ChanLoad<T, G>& L, float (&acc)[kNB][G],
                                             float& o, F&& issue_next) {
  constexpr uint32_t x0 = 0x3C00u >> T;
  uint32_t x[kNB];
  x[0] = shift_in_plane(x0, L.pw[0][0]);
  __builtin_amdgcn_sched_barrier(0);
  issue_next();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 1; b < kNB; ++b) x[b] = shift_in_plane(x0, L.pw[0][b]);
#pragma unroll
  for (int p = 1; p < T; ++p)
#pragma unroll
    for (int b = 0; b < kNB; ++b) x[b] = shift_in_plane(x[b], L.pw[p][b]);
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const uint32_t ab = (b & 1) ? (L.a2[b >> 1] >> 16) : L.a2[b >> 1];
    const float a = half_lo(ab);
    const float m = __builtin_fmaf(a, half_lo(x[b]), -a);
#pragma unroll
    for (int h = 0; h < G; ++h) acc[b][h] = __builtin_fmaf(L.w[h], m, acc[b][h]);
  }
  o = __builtin_fmaf(L.e, half_lo(L.oa), o);
}

template <int T, int G>
__device__ __forceinline__ void compute_chan(const ChanLoad<T, G>& L, float (&acc)[kNB][G],
                                             float& o) {
  compute_chan<T, G>(L, acc, o, [] {});
}

// Epilogue: S = U + o (o of block b, head h sits in lane b * G + h); blocks
// [store_from, store_to] of the tile are stored.
template <int G>
__device__ __forceinline__ void store_tile(const float (&acc)[kNB][G], float o, int store_from,
                                           int store_to, int64_t n, float* __restrict__ out) {
  const int lane = lane_id();
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    if (b >= store_from && b <= store_to) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float obh = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, o), b * G + h));
        __builtin_nontemporal_store(acc[b][h] + obh, out + h * n + b * kBlock + lane);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Main kernel: whole rounds, L2 prefetch, scales staged in LDS
// ---------------------------------------------------------------------------

template <int G>
struct MainShared {
  GroupTables<G> tb;
  alignas(16) uint16_t sc[2][kSlots][kRoundBlocks];   // staged block scales, two rounds
};

struct MainTile {
  const char* planes;       // the group's plane rows at the tile's first block
  uint32_t pstride;         // bytes between two planes of a channel
  const uint16_t* sc;       // staged scales of the round, at the tile's first block
  int ob;                   // this lane's block in the offset fold
  int oh;                   // this lane's head in the offset fold
};

template <int T, int G>
__device__ __forceinline__ void main_load(const MainTile& c, const GroupTables<G>& tb, int slot,
                                          uint32_t off, ChanLoad<T, G>& L) {
  const char* rp = c.planes + off;
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int b = 0; b < kNB; ++b)
      L.pw[p][b] = *reinterpret_cast<const uint64_t*>(rp + p * c.pstride + b * 8);
  const uint16_t* sp = c.sc + slot * kRoundBlocks;
#pragma unroll
  for (int i = 0; i < kNB / 2; ++i) L.a2[i] = reinterpret_cast<const uint32_t*>(sp)[i];
#pragma unroll
  for (int h = 0; h < G; ++h) L.w[h] = tb.w[slot][h];
  L.e = tb.e[slot][c.oh];
  L.oa = sp[c.ob];
  L.noff = tb.poff[slot + 1];
}

// The channels of depth T: active slots [first, first + cnt).  Two register
// sets alternate; the loads of slot i + 1 are issued while slot i is
// computed.  The pipeline reads up to two slots past the range (padding or
// other active channels), which are never computed.
template <int T, int G>
__device__ __forceinline__ void main_depth(const MainTile& c, const GroupTables<G>& tb, int first,
                                           int cnt, float (&acc)[kNB][G], float& o) {
  if (cnt <= 0) return;
  ChanLoad<T, G> A, B;
  main_load<T, G>(c, tb, first, uniform(tb.poff[first]), A);
  int i = 0;
  for (; i + 1 < cnt; i += 2) {
    compute_chan<T, G>(A, acc, o, [&] { main_load<T, G>(c, tb, first + i + 1, uniform(A.noff), B); });
    compute_chan<T, G>(B, acc, o, [&] { main_load<T, G>(c, tb, first + i + 2, uniform(B.noff), A); });
  }
  if (i < cnt) compute_chan<T, G>(A, acc, o);
}

// The vector loads of one round: the scales of every active slot (kept in
// registers until the round is staged) and two touches (at +0 and +64 bytes)
// of every active plane row's 128-byte segment, which pull the lines into L2
// ahead of the scalar loads.  A16: scale rows are 16-byte aligned (capacity a
// multiple of 8 blocks), so a slot's 16 scales are two 16-byte loads;
// otherwise 8 halves per thread are loaded one by one.
constexpr int kThreads = kWaves * 64;
constexpr int kRowsPerThread = kD * kPlanes / kThreads;             // 2
template <bool A16>
struct Stage {
  static constexpr int kWords = A16 ? 4 : kD * kRoundBlocks / kThreads;   // 4 or 8
  uint32_t st[kWords];
  uint32_t tv[2 * kRowsPerThread];
};

template <int G, bool A16>
__device__ __forceinline__ void round_issue(const GroupTables<G>& tb, const char* planes_g,
                                            const char* scales_g, int64_t r0, Stage<A16>& S) {
  const int tid = threadIdx.x;
  if (A16) {
    const int slot = tid >> 1, half = tid & 1;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    // poff / 16 = j * nb_store * 2: the byte offset of channel j's scale row.
    if (slot < tb.nact)
      v = *reinterpret_cast<const uint4*>(scales_g + (tb.poff[slot] >> 4) + r0 * 2 + half * 16);
    S.st[0] = v.x; S.st[1] = v.y; S.st[2] = v.z; S.st[3] = v.w;
  } else {
    const int nst = tb.nact * kRoundBlocks;
#pragma unroll
    for (int i = 0; i < Stage<A16>::kWords; ++i) {
      const int k = tid + i * kThreads;
      S.st[i] = 0u;
      if (k < nst) {
        const int slot = k / kRoundBlocks, b = k % kRoundBlocks;
        S.st[i] = *reinterpret_cast<const uint16_t*>(scales_g + (tb.poff[slot] >> 4) + (r0 + b) * 2);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRowsPerThread; ++i) {
    const int k = tid + i * kThreads;
    S.tv[2 * i] = S.tv[2 * i + 1] = 0u;
    if (k < tb.nrows) {
      const char* rp = planes_g + tb.prow[k] + r0 * 8;
      S.tv[2 * i] = *reinterpret_cast<const uint32_t*>(rp);
      S.tv[2 * i + 1] = *reinterpret_cast<const uint32_t*>(rp + 64);
    }
  }
}

// Write a round's scales to LDS and retire its L2 touches (their values are
// folded into `sink`, which only keeps the loads from being dropped).
template <int G, bool A16>
__device__ __forceinline__ void round_stage(MainShared<G>& sh, int buf, const Stage<A16>& S,
                                            uint32_t& sink) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2 * kRowsPerThread; ++i) sink ^= S.tv[i];
  if (A16) {
    const int slot = tid >> 1, half = tid & 1;
    if (slot < sh.tb.nact)
      *reinterpret_cast<uint4*>(&sh.sc[buf][slot][half * 8]) = make_uint4(S.st[0], S.st[1], S.st[2], S.st[3]);
  } else {
    const int nst = sh.tb.nact * kRoundBlocks;
#pragma unroll
    for (int i = 0; i < Stage<A16>::kWords; ++i) {
      const int k = tid + i * kThreads;
      if (k < nst) sh.sc[buf][k / kRoundBlocks][k % kRoundBlocks] = (uint16_t)S.st[i];
    }
  }
}

template <int G, bool A16>
__global__ __launch_bounds__(kWaves * 64) void scan_main(
    const uint64_t* __restrict__ planes, const uint16_t* __restrict__ scales, int64_t nb_store,
    const uint8_t* __restrict__ depths, const float* __restrict__ q, int64_t nrounds, int64_t n,
    int64_t wgs_per_group, float* __restrict__ scores) {
  static_assert(kNB * G <= 64, "one lane per (block, head) in the offset fold");
  __shared__ MainShared<G> sh;
  GroupTables<G>& tb = sh.tb;

  // XCD-aware remap of the workgroup id (bijective on [0, gridDim.x)).
  const uint32_t nwg = gridDim.x;
  const uint32_t per_xcd = nwg / kXcds;
  uint32_t id = blockIdx.x;
  if (id < per_xcd * kXcds) id = (id % kXcds) * per_xcd + id / kXcds;
  const int64_t grp = id / wgs_per_group;
  const int64_t round0 = (id % wgs_per_group) * kRounds;
  const int nr = (int)min<int64_t>(kRounds, nrounds - round0);

  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t pstride = (uint32_t)nb_store * 8u;
  const char* planes_g =
      reinterpret_cast<const char*>(planes + grp * kD * (int64_t)kPlanes * nb_store);
  const char* scales_g = reinterpret_cast<const char*>(scales + grp * kD * nb_store);
  float* scores_g = scores + grp * G * n;

  build_tables<G>(tb, depths, q, grp, pstride);
  __syncthreads();

  uint32_t sink = 0u;
  Stage<A16> S;
  round_issue<G, A16>(tb, planes_g, scales_g, round0 * kRoundBlocks, S);
  round_stage<G, A16>(sh, 0, S, sink);
  __syncthreads();

  const bool olane = lane < kNB * G;
  MainTile c;
  c.pstride = pstride;
  c.ob = olane ? lane / G : 0;
  c.oh = olane ? lane % G : 0;
  const int c4 = tb.count[0], c3 = tb.count[1], c2 = tb.count[2], c1 = tb.count[3];

  for (int r = 0; r < nr; ++r) {
    const int64_t r0 = (round0 + r) * kRoundBlocks;
    if (r + 1 < nr) round_issue<G, A16>(tb, planes_g, scales_g, r0 + kRoundBlocks, S);

    const int64_t blk0 = r0 + wave * kNB;
    c.planes = planes_g + blk0 * 8;
    c.sc = &sh.sc[r & 1][0][wave * kNB];
    float acc[kNB][G];
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
      for (int h = 0; h < G; ++h) acc[b][h] = 0.0f;
    float o = 0.0f;
    main_depth<4, G>(c, tb, 0, c4, acc, o);
    main_depth<3, G>(c, tb, c4, c3, acc, o);
    main_depth<2, G>(c, tb, c4 + c3, c2, acc, o);
    main_depth<1, G>(c, tb, c4 + c3 + c2, c1, acc, o);
    store_tile<G>(acc, o, 0, kNB - 1, n, scores_g + blk0 * kBlock);

    if (r + 1 < nr) round_stage<G, A16>(sh, (r + 1) & 1, S, sink);
    __syncthreads();
  }
  asm volatile("" ::"v"(sink));   // keeps the L2 touches alive
}

// ---------------------------------------------------------------------------
// Tail kernel: per-block clamped loads, blocks [first_blk, nblk) of a group
// ---------------------------------------------------------------------------

struct TailTile {
  const uint64_t* planes;   // the group's plane rows
  const uint16_t* scales;   // the group's scale rows
  int64_t nb_store;
  int64_t blk0;             // first block of the tile
  int last;                 // last valid block offset in the tile
  int ob_c;                 // this lane's block in the offset fold (clamped)
  int oh;                   // this lane's head in the offset fold
};

// The tail kernel builds its tables with pstride = 8, so poff = 32 * j names
// the channel; offsets are then formed in 64 bits.
template <int T, int G>
__device__ __forceinline__ void tail_load(const TailTile& c, const GroupTables<G>& tb, int slot,
                                          ChanLoad<T, G>& L) {
  const int64_t j = (int64_t)(tb.poff[slot] / (kPlanes * 8));
  const uint64_t* rp = c.planes + j * kPlanes * c.nb_store + c.blk0;
#pragma unroll
  for (int p = 0; p < T; ++p)
#pragma unroll
    for (int b = 0; b < kNB; ++b) L.pw[p][b] = rp[p * c.nb_store + min(b, c.last)];
  const uint16_t* sp = c.scales + j * c.nb_store + c.blk0;
#pragma unroll
  for (int i = 0; i < kNB / 2; ++i)
    L.a2[i] = (uint32_t)sp[min(2 * i, c.last)] | ((uint32_t)sp[min(2 * i + 1, c.last)] << 16);
#pragma unroll
  for (int h = 0; h < G; ++h) L.w[h] = tb.w[slot][h];
  L.e = tb.e[slot][c.oh];
  L.oa = sp[c.ob_c];
}

template <int T, int G>
__device__ __forceinline__ void tail_depth(const TailTile& c, const GroupTables<G>& tb, int first,
                                           int cnt, float (&acc)[kNB][G], float& o) {
  for (int i = 0; i < cnt; ++i) {
    ChanLoad<T, G> L;
    tail_load<T, G>(c, tb, first + i, L);
    compute_chan<T, G>(L, acc, o);
  }
}

template <int G>
__global__ __launch_bounds__(kWaves * 64) void scan_tail(
    const uint64_t* __restrict__ planes, const uint16_t* __restrict__ scales, int64_t nb_store,
    const uint8_t* __restrict__ depths, const float* __restrict__ q, int64_t first_blk,
    int64_t nblk, int64_t n, int64_t wgs_per_group, float* __restrict__ scores) {
  __shared__ GroupTables<G> tb;
  const int64_t grp = blockIdx.x / wgs_per_group;
  const int64_t wg = blockIdx.x % wgs_per_group;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  build_tables<G>(tb, depths, q, grp, 8u);
  __syncthreads();

  TailTile c;
  c.planes = planes + grp * kD * (int64_t)kPlanes * nb_store;
  c.scales = scales + grp * kD * nb_store;
  c.nb_store = nb_store;
  const bool olane = lane < kNB * G;
  const int ob = olane ? lane / G : 0;
  c.oh = olane ? lane % G : 0;
  c.blk0 = first_blk + (wg * kWaves + wave) * kNB;
  if (c.blk0 >= nblk) return;
  c.last = (int)min<int64_t>(kNB, nblk - c.blk0) - 1;
  c.ob_c = min(ob, c.last);

  float acc[kNB][G];
#pragma unroll
  for (int b = 0; b < kNB; ++b)
#pragma unroll
    for (int h = 0; h < G; ++h) acc[b][h] = 0.0f;
  float o = 0.0f;
  const int c4 = tb.count[0], c3 = tb.count[1], c2 = tb.count[2], c1 = tb.count[3];
  tail_depth<4, G>(c, tb, 0, c4, acc, o);
  tail_depth<3, G>(c, tb, c4, c3, acc, o);
  tail_depth<2, G>(c, tb, c4 + c3, c2, acc, o);
  tail_depth<1, G>(c, tb, c4 + c3 + c2, c1, acc, o);
  store_tile<G>(acc, o, 0, c.last, n, scores + grp * G * n + c.blk0 * kBlock);
}

template <int G>
void launch_scan_g(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                   const uint8_t* depths, const float* q, int64_t groups, int64_t n,
                   float* scores, hipStream_t stream) {
  const int64_t nblk = n / kBlock;
  const bool fast = nb_store <= kMaxFastBlocks;
  const int64_t nrounds = fast ? nblk / kRoundBlocks : 0;
  if (nrounds > 0) {
    const int64_t wgs = (nrounds + kRounds - 1) / kRounds;
    const dim3 grid((unsigned)(wgs * groups)), block(kWaves * 64);
    if (nb_store % 8 == 0 && (reinterpret_cast<uintptr_t>(scales) & 15) == 0)
      hipLaunchKernelGGL((scan_main<G, true>), grid, block, 0, stream, planes, scales, nb_store,
                         depths, q, nrounds, n, wgs, scores);
    else
      hipLaunchKernelGGL((scan_main<G, false>), grid, block, 0, stream, planes, scales, nb_store,
                         depths, q, nrounds, n, wgs, scores);
  }
  const int64_t first = nrounds * kRoundBlocks;
  if (first < nblk) {
    const int64_t wgs = (nblk - first + kRoundBlocks - 1) / kRoundBlocks;
    hipLaunchKernelGGL(scan_tail<G>, dim3((unsigned)(wgs * groups)), dim3(kWaves * 64), 0, stream,
                       planes, scales, nb_store, depths, q, first, nblk, n, wgs, scores);
  }
}

}  // namespace

int64_t scan_max_workgroups(int64_t groups, int64_t n) {
  const int64_t nblk = n / kBlock;
  return groups * ((nblk + kRoundBlocks - 1) / kRoundBlocks);
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
