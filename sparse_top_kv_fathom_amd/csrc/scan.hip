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
//   o_hb = fold_j fma(e_hj, a_bj, o),   o from +0,  e_hj = fl32(q_hj * (2^-t_j - 1)),
//   U_hi = fold_j fma(w_hj, m_ij, U),   U from +0,  w_hj = q_hj * 2^(11-t_j),
//                                                    m_ij = a_bj * c'_ij * 2^-10,
//   S_hi = fl32(U_hi + o_hb),
// both folds over the active channels, deepest first and by ascending index
// within a depth.  w and m are exact, so every fold step rounds once.
//
// Mapping.  A wave owns a tile of kNB = 8 consecutive 64-token blocks; lane i
// is token i of every block, i.e. bit i of every plane word.  The 8 plane
// words of one (channel, plane) are one 64-byte scalar load, and a word is
// used directly as the per-lane carry-in of v_addc_co_u32, so plane p of a
// block costs one VALU instruction:  x <- 2x + bit_p.  Starting from
// 0x3F800000 >> t, t steps leave x = 0x3F800000 + c', the fp32 pattern of
// 1 + c' * 2^-23, and one fp32 FMA with the block scale staged as
// A = a * 2^13 gives m = A * x - A = a * c' * 2^-10 exactly (all operands in
// vector registers, which issue faster than the mixed-precision form).  Each head
// then costs one fp32 FMA: t + 1 + G VALU instructions per channel and
// block.  At depth 1, m is 0 or a * 2^-10 (staged as such): one select with
// the plane word as its lane mask, then the G head FMAs (fma(w, +0, U) = U,
// as U is never -0): 1 + G instructions.  The block offsets o fold on 8 * G
// lanes (lane = block * G + head), one instruction per channel, and are added
// in the epilogue.
//
// Resources.  The scalar-load path of gfx950 moves only a few bytes per clock
// per CU, so it carries nothing but plane words (the bytes the method reads).
// Weights, offset coefficients and block scales come from LDS: w and e per
// active channel once per workgroup, the scales of every active channel once
// per round of kRoundBlocks blocks (staged with vector loads, stored in LDS
// as fp32 A = a * 2^13, or a * 2^-10 for depth-1 channels).
//
// Latency.  A workgroup reads the plan and the queries in one round trip,
// then loads its round's scales and touches every plane line of the round with
// vector loads (one 4-byte load per 128-byte line pulls the line into L2); it
// waits for the scales only and computes while the touches are in flight, so
// its scalar loads hit L2 or a fill already on its way.  (Touching a round ahead while computing the current one keeps twice
// the lines in flight and they are evicted from the 4 MB L2 of an XCD before
// use; one round per workgroup measured fastest.)  Channels of one
// depth form a loop with a compile-time plane count.  Scalar loads return out
// of order, so the only usable wait is "all outstanding"; for depths 1 and 2
// two register sets alternate and each channel waits once, at its first
// instruction, before it issues the next channel's loads, which then overlap
// its arithmetic.  Depths 3 and 4 (64-128 plane registers) load and compute
// one at a time.
//
// Grid.  Main kernel: whole rounds only (4 waves, 32 blocks, 2048 tokens per
// workgroup; 8-wave workgroups measured the same), workgroup ids remapped so
// that consecutive rounds of a group run on the same XCD (workgroups are
// dealt to the 8 XCDs round-robin).  The blocks after the last whole round
// go to a small tail kernel (one workgroup per 512-token tile, staged in
// LDS), which also serves groups whose plane array needs 64-bit offsets.
#include <hip/hip_ext.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <type_traits>

#include "fathom_internal.h"
#include "topk_layout.h"
#include "topk_select.h"

// Compile-time tuning: SCAN_U1 = depth-1 channels per pipelined set,
// SCAN_ROUNDS = rounds per workgroup, SCAN_TOUCHES = L2 touches per 256-byte
// plane-row segment of a round.
#ifndef SCAN_U1
#define SCAN_U1 1
#endif

namespace fathom {
namespace {

constexpr int kWaves = 4;                    // waves per workgroup
constexpr int kThreads = kWaves * 64;
constexpr int kNB = 8;                       // blocks per wave tile (512 tokens)
constexpr int kRoundBlocks = kWaves * kNB;   // blocks per workgroup round
#ifndef SCAN_ROUNDS
#define SCAN_ROUNDS 1
#endif
constexpr int kRounds = SCAN_ROUNDS;         // rounds per workgroup (main kernel)
constexpr int kXcds = 8;
constexpr int kSlots = kD + 4;               // active slots + padding read by the pipeline
// Byte offsets inside one group's plane array are 32-bit in the main kernel.
constexpr int64_t kMaxFastBlocks = (int64_t(1) << 32) / (kD * kPlanes * 8) - 1;

// x <- 2x + (bit lane of mask): the plane word is the carry-in lane mask.
// The carry-out (always 0 here: x < 2^31) goes to a scratch scalar pair, not
// to VCC: a stream of these adds interleaved with fp32 FMAs issues about a
// third faster when they do not write VCC.
__device__ __forceinline__ uint32_t shift_in_plane(uint32_t x, uint64_t mask) {
  uint32_t r;
  uint64_t co;
  asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=&s"(co) : "v"(x), "s"(mask));
  return r;
}
// The same as a volatile statement: it stays in program order with the other
// volatile statements (the first instruction of a channel, which carries the
// wait for that channel's loads).
__device__ __forceinline__ uint32_t shift_in_plane_ordered(uint32_t x, uint64_t mask) {
  uint32_t r;
  uint64_t co;
  asm volatile("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=&s"(co) : "v"(x), "s"(mask));
  return r;
}

// Make a value opaque to the optimizer at this point, so that work derived
// from it is redone here instead of being hoisted (and held in registers)
// across a loop.
__device__ __forceinline__ void opaque_s(uint64_t& v) { asm volatile("" : "+s"(v)); }
__device__ __forceinline__ void opaque_s(int& v) { asm volatile("" : "+s"(v)); }
__device__ __forceinline__ void opaque_v(int& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ float half_lo(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits & 0xffffu));
}

// Active channels of a group: one 128-bit mask per depth (bit j set when
// t_j equals that depth), built by every wave from the depth row with ballots.
struct DepthMasks {
  uint64_t lo[kPlanes], hi[kPlanes];   // index 0: depth 4, ... 3: depth 1
  int count[kPlanes];
  int tlo, thi;                        // depths of channels lane and 64 + lane
};

__device__ __forceinline__ DepthMasks depth_masks(int dlo, int dhi) {
  const int tlo = min(dlo, kPlanes);   // depths above 4 read as 4
  const int thi = min(dhi, kPlanes);
  DepthMasks m;
  m.tlo = tlo;
  m.thi = thi;
#pragma unroll
  for (int i = 0; i < kPlanes; ++i) {
    m.lo[i] = __ballot(tlo == kPlanes - i);
    m.hi[i] = __ballot(thi == kPlanes - i);
    m.count[i] = __popcll(m.lo[i]) + __popcll(m.hi[i]);
  }
  return m;
}

// Ascending iteration over the set bits of a 128-bit wave-uniform mask;
// returns channel 0 once the mask is empty (reads past the end stay valid).
struct ChanIter {
  uint64_t lo, hi;
  __device__ __forceinline__ int next() {
    int j = 0;
    if (lo != 0) {
      j = __builtin_ctzll(lo);
      lo &= lo - 1;
    } else if (hi != 0) {
      j = 64 + __builtin_ctzll(hi);
      hi &= hi - 1;
    }
    return j;
  }
};

// Everything one channel contributes to a wave tile.
template <int T, int G>
struct ChanLoad {
  uint64_t pw[T][kNB];    // plane words (wave-uniform)
  float A[kNB];           // block scales as a * 2^13; a * 2^-10 at depth 1 (same in every lane)
  float w[G];             // per-head weights (same in every lane)
  float e;                // offset coefficient of this lane's head
  float oa;               // the scale of this lane's block as in A (offset fold)
};

// m = A in the lanes whose bit is set in the plane word `mask`, +0 in the
// others (one select with the word as its lane mask).  The _ordered form is
// a volatile statement, so it stays where it is written when it opens a
// channel (it carries the wait for the channel's loads).
__device__ __forceinline__ float select_plane(uint64_t mask, float A) {
  float m;
  asm("v_cndmask_b32_e64 %0, 0, %1, %2" : "=v"(m) : "v"(A), "s"(mask));
  return m;
}
__device__ __forceinline__ float select_plane_ordered(uint64_t mask, float A) {
  float m;
  asm volatile("v_cndmask_b32_e64 %0, 0, %1, %2" : "=v"(m) : "v"(A), "s"(mask));
  return m;
}

// Channel of depth T for the wave tile.  `issue_next` runs right after the
// first instruction that reads this channel's registers (which carries the
// wait for everything outstanding), so the next channel's loads overlap the
// rest of this one; scheduling barriers keep the compiler from moving work
// across that point.
template <int T, int G, class F>
__device__ __forceinline__ void compute_chan(const ChanLoad<T, G>& L, float (&acc)[kNB][G],
                                             float& o, F&& issue_next) {
  if constexpr (T == 1) {
    // Depth 1: c' is the plane bit, so m = a * c' * 2^-10 is either 0 or
    // a * 2^-10 (staged as A for depth-1 channels): one select with the plane
    // word as the lane mask gives m, the same value the general form computes
    // in two steps.
    __builtin_amdgcn_sched_barrier(0);
    const float m0 = select_plane_ordered(L.pw[0][0], L.A[0]);   // waits for the loads
    __builtin_amdgcn_sched_barrier(0);
    issue_next();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < G; ++h) acc[0][h] = __builtin_fmaf(L.w[h], m0, acc[0][h]);
#pragma unroll
    for (int b = 1; b < kNB; ++b) {
      const float m = select_plane(L.pw[0][b], L.A[b]);
#pragma unroll
      for (int h = 0; h < G; ++h) acc[b][h] = __builtin_fmaf(L.w[h], m, acc[b][h]);
    }
    o = __builtin_fmaf(L.e, __builtin_ldexpf(L.oa, 10), o);
    asm volatile("" : "+v"(o));
    return;
  }
  constexpr uint32_t x0 = 0x3F800000u >> T;
  uint32_t x[kNB];
  // The first instruction waits for this channel's loads; it must not move
  // above the previous channel's arithmetic, which hides their latency (the
  // accumulators are pinned at the end of every channel below).
  __builtin_amdgcn_sched_barrier(0);
  x[0] = shift_in_plane_ordered(x0, L.pw[0][0]);
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
    const float m = __builtin_fmaf(L.A[b], __builtin_bit_cast(float, x[b]), -L.A[b]);
#pragma unroll
    for (int h = 0; h < G; ++h) acc[b][h] = __builtin_fmaf(L.w[h], m, acc[b][h]);
  }
  o = __builtin_fmaf(L.e, __builtin_ldexpf(L.oa, -13), o);
#pragma unroll
  for (int b = 0; b < kNB; ++b)
#pragma unroll
    for (int h = 0; h < G; ++h) asm volatile("" : "+v"(acc[b][h]));
  asm volatile("" : "+v"(o));
}

// Epilogue: S = U + o (o of block b, head h sits in lane b * G + h), left in
// acc; blocks [0, store_to] of the tile are stored when `out` is non-null.
// The offsets pass through the wave's own kNB * G floats of LDS (`s_o`) and
// come back as broadcast reads, so the adds take vector operands (dual issue)
// instead of one lane read and one scalar-operand add per (block, head).
template <int G>
__device__ __forceinline__ void finish_tile(float (&acc)[kNB][G], float o, int store_to, int64_t n,
                                            float* __restrict__ out, float* s_o) {
  const int lane = lane_id();
  if (lane < kNB * G) s_o[lane] = o;
  wave_lds_sync();
#pragma unroll
  for (int b = 0; b < kNB; ++b)
#pragma unroll
    for (int h = 0; h < G; ++h) acc[b][h] = acc[b][h] + s_o[b * G + h];
  if (out != nullptr) {
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      if (b <= store_to) {
#pragma unroll
        for (int h = 0; h < G; ++h)
          __builtin_nontemporal_store(acc[b][h], out + h * n + b * kBlock + lane);
      }
    }
  }
}

// Candidates of fathom_scan_topk.  Each wave tile (kNB blocks = kTileKeys
// keys of a row) owns `region` slots of the row's candidate buffer, at slot
// tile * region; the main kernel pools the slots of a round's kWaves tiles
// (emit_round), the tail kernel fills each tile's own.  The segment table
// holds, per tile, the first slot of its candidates and their count; every
// score >= tau of head h goes there as (order key, index), in index order.
constexpr int kTileKeys = kNB * kBlock;
constexpr int64_t kFusedMinKeys = 65536;   // shorter rows: scan, then top-k
constexpr int64_t kFusedMaxTiles = 4096;   // regions per row the selection stages
constexpr int kRescanRounds = 8;           // rounds per workgroup of the gated second pass
constexpr int kSampleRuns = 8;             // sampled runs of two wave tiles per group
constexpr int kSampleKeys = 2 * kSampleRuns * kTileKeys;   // 8192 per row
constexpr int kSampleWgBlocks = 4;                         // blocks per sample workgroup
constexpr int kSampleWgs = 2 * kSampleRuns * kNB / kSampleWgBlocks;   // per group (32)
constexpr int kCutSpin = 2048;             // polls (about 0.2 us each) of a cut not yet out

// The sample and the cut of fathom_scan_topk, taken inside the candidate
// scan's launch.  Its first groups * kSampleWgs workgroups (a multiple of the
// XCD count, so the scan's own ids keep their XCD) each score four blocks of
// the group's sample: 8 runs of two adjacent wave tiles spread evenly over
// the row.  Their order keys go to the sample buffer with agent-scope stores,
// and each workgroup then sets its own flag to the call's epoch.  Sample
// workgroups 0 to G - 1 of a group wait until all the group's flags carry
// this call's epoch and take one row's cut each: tau = the target-th largest of the
// row's kSampleKeys sampled keys with its low 10 bits cleared (two 11-bit
// radix digits, the keys read with agent-scope loads), stored for the
// selection and published in the row's ready word as tau | epoch << 1 | 1
// with an agent-scope atomic store.  Every message is a single word or is
// complete before the word that announces it is written (s_waitcnt), so no
// fence is needed (a device-scope release would write back the L2).
// Scan waves read the ready word with agent-scope loads before their depth-1
// channels and poll it (boundedly) only if this call's cut is not out yet; a
// cut still missing after `spin` polls flags the row, and every emitting tile
// stamps the cut it used, which the selection checks, so that no timing or
// stale word can change a result: it can only send a row to the fallback.
struct CutArgs {
  uint32_t* sample;         // [rows][kMaxSampleKeys] sampled order keys
  int target;               // rank of tau among the row's kSampleKeys keys
  int groups;               // groups sampled; 0 outside the candidate scan
  topk::RowGeom geom;       // the rows' selection state (R = kTileKeys)
  int publish;              // 1; 0 only under fathom_test_cut_hooks
  int spin;                 // the waves' poll limit (kCutSpin)
  int64_t rstride;          // wave tiles between two sampled runs
  uint32_t* gflag;          // [groups] second-pass flags (cleared by the cut)
  uint32_t* sflag;          // [groups][kSampleFlags] epochs of the sample parts that are out
  uint32_t epoch;           // the call's epoch (its low 9 bits are used)
};

__host__ __device__ inline uint32_t sample_workgroups(int groups) {
  static_assert((kSampleWgs % kXcds) == 0, "whole XCD rounds");
  static_assert(kSampleWgs <= topk::kSampleFlags, "one flag per sample workgroup, one per lane");
  return (uint32_t)groups * kSampleWgs;
}
// The low 10 bits of a published ready word.
__device__ __forceinline__ uint32_t ready_bits(uint32_t epoch) { return ((epoch & 0x1FFu) << 1) | 1u; }

// The sample's channels of depth T (mask m over 64 channels from c0) for
// lane `bit` of half `hsel` of block `b`, four at a time: the
// LDS reads of the four (the lane's T plane words in one read, the scale,
// the G query entries in one read) are issued together, then their
// arithmetic.  A slot past the end of the mask reads channel c0 and adds 0.
template <int T, int G>
__device__ __forceinline__ void sample_depth(const uint4 (*s_w)[kSampleWgBlocks][2],
                                             const uint16_t (*s_sc)[kSampleWgBlocks],
                                             const float (*s_q)[G], uint64_t m, int c0, int b,
                                             int hsel, int bit, float (&acc)[G]) {
  while (m != 0ull) {
    int c[4];
    bool ok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ok[u] = m != 0ull;
      c[u] = c0 + (ok[u] ? __builtin_ctzll(m) : 0);
      m &= m - 1;   // stays 0 once empty
    }
    uint32_t w[4][T];
    float a[4], qv[4][G];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // Word hsel of planes 0-3 of channel c, block b.
      const uint32_t* wp = reinterpret_cast<const uint32_t*>(&s_w[c[u]][b][hsel]);
#pragma unroll
      for (int p = 0; p < T; ++p) w[u][p] = wp[p];
      a[u] = half_lo(s_sc[c[u]][b]);
#pragma unroll
      for (int h = 0; h < G; ++h) qv[u][h] = s_q[c[u]][h];   // uniform address: broadcast
    }
    __builtin_amdgcn_sched_barrier(0);   // every read above is issued before the arithmetic
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t cp = 0u;
#pragma unroll
      for (int p = 0; p < T; ++p) cp = 2 * cp + ((w[u][p] >> bit) & 1u);
      // (c' + 1/2 - 2^(T-1)) * a / 2^(T-1)
      float kh = __builtin_ldexpf(((float)cp + (0.5f - (float)(1 << (T - 1)))) * a[u], 1 - T);
      kh = ok[u] ? kh : 0.0f;
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = __builtin_fmaf(qv[u][h], kh, acc[h]);
    }
  }
}

// One sample workgroup of the candidate scan (workgroup id `wg` below
// sample_workgroups): blocks 4 pr to 4 pr + 3 of sampled tile ti, in fp32
// but in no particular order (only the cut is taken from the sample).  One
// round of loads brings the depths, the blocks' scales, the group's queries
// and every plane row of the blocks (512 rows of 32 bytes, the rows past a
// channel's depth too, so no load waits for the plan) into LDS, laid out so
// that a lane reads its channel's plane words, and a channel's query
// entries, in one LDS read each; wave b scores block b over every active
// channel.  Then its flag and, in sample workgroups 0 to G - 1, a cut.
template <int G>
__device__ void sample_wg(const CutArgs& cut, uint32_t wg, const uint64_t* __restrict__ planes,
                          const uint16_t* __restrict__ scales, int64_t nb_store,
                          const uint8_t* __restrict__ depths, const float* __restrict__ q,
                          void* tws, char* smem) {
  constexpr int SB = kSampleWgBlocks;
  static_assert(SB == kWaves, "one wave per block");
  constexpr int kScOff = kD * SB * 2 * 16;
  constexpr int kQOff = kScOff + kD * SB * 2;                // after s_w and s_sc
  constexpr int kArrOff = kQOff + kD * G * 4;
  static_assert(kQOff % 16 == 0, "s_q in whole 16-byte rows");
  uint4 (*s_w)[SB][2] = reinterpret_cast<uint4 (*)[SB][2]>(smem);             // [kD][SB][2]
  uint16_t (*s_sc)[SB] = reinterpret_cast<uint16_t (*)[SB]>(smem + kScOff);
  float (*s_q)[G] = reinterpret_cast<float (*)[G]>(smem + kQOff);
  uint32_t* s_arr = reinterpret_cast<uint32_t*>(smem + kArrOff);
  const int64_t grp = wg / kSampleWgs;
  const int sb = (int)(wg % kSampleWgs);
  constexpr int kPerTile = kNB / SB;                          // sample workgroups per tile
  const int ti = sb / kPerTile, pr = sb % kPerTile;
  const int64_t blk0 = ((ti >> 1) * cut.rstride + (ti & 1)) * kNB + SB * pr;
  const int tid = threadIdx.x, lane = lane_id();
  const int b = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's block
  const int tlo = min((int)depths[grp * kD + lane], kPlanes);
  const int thi = min((int)depths[grp * kD + 64 + lane], kPlanes);
  for (int i = tid; i < G * kD; i += kThreads) s_q[i % kD][i / kD] = q[grp * G * kD + i];
  if (tid < kD) {
    const uint16_t* sp = scales + (grp * kD + tid) * nb_store + blk0;
#pragma unroll
    for (int u = 0; u < SB; ++u) s_sc[tid][u] = sp[u];
  }
  // Plane rows r = tid and tid + 256: (channel r / 4, plane r % 4), the
  // workgroup's SB blocks.
  const bool vec = (nb_store & 1) == 0 && (reinterpret_cast<uintptr_t>(planes) & 15) == 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = tid + kThreads * i;
    const uint64_t* a0 = planes + (grp * kD * kPlanes + r) * nb_store + blk0;
    uint64_t x[SB];
    if (vec) {
#pragma unroll
      for (int u = 0; u < SB / 2; ++u) {
        const uint4 v = reinterpret_cast<const uint4*>(a0)[u];
        x[2 * u] = v.x | ((uint64_t)v.y << 32);
        x[2 * u + 1] = v.z | ((uint64_t)v.w << 32);
      }
    } else {
#pragma unroll
      for (int u = 0; u < SB; ++u) x[u] = a0[u];
    }
    uint32_t* w = reinterpret_cast<uint32_t*>(s_w[r >> 2][0]) + (r & 3);
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      w[8 * u] = (uint32_t)x[u];               // block u, tokens 0-31
      w[8 * u + 4] = (uint32_t)(x[u] >> 32);   //          tokens 32-63
    }
  }
  __syncthreads();
  const int hsel = lane >> 5, bit = lane & 31;
  float acc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h] = 0.0f;
  sample_depth<4, G>(s_w, s_sc, s_q, __ballot(tlo == 4), 0, b, hsel, bit, acc);
  sample_depth<4, G>(s_w, s_sc, s_q, __ballot(thi == 4), 64, b, hsel, bit, acc);
  sample_depth<3, G>(s_w, s_sc, s_q, __ballot(tlo == 3), 0, b, hsel, bit, acc);
  sample_depth<3, G>(s_w, s_sc, s_q, __ballot(thi == 3), 64, b, hsel, bit, acc);
  sample_depth<2, G>(s_w, s_sc, s_q, __ballot(tlo == 2), 0, b, hsel, bit, acc);
  sample_depth<2, G>(s_w, s_sc, s_q, __ballot(thi == 2), 64, b, hsel, bit, acc);
  sample_depth<1, G>(s_w, s_sc, s_q, __ballot(tlo == 1), 0, b, hsel, bit, acc);
  sample_depth<1, G>(s_w, s_sc, s_q, __ballot(thi == 1), 64, b, hsel, bit, acc);
#pragma unroll
  for (int h = 0; h < G; ++h)
    __hip_atomic_store(cut.sample + (grp * G + h) * (int64_t)topk::kMaxSampleKeys +
                           ti * kTileKeys + (SB * pr + b) * kBlock + lane,
                       topk::order_key(acc[h]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the keys are out before the flag
  __syncthreads();
  uint32_t* flags = cut.sflag + grp * topk::kSampleFlags;
  if (tid == 0) __hip_atomic_store(flags + sb, cut.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (sb >= G) return;   // uniform over the workgroup
  const int h = sb;
  // Wave 0 reads the group's flags, one per lane, until all are this call's.
  if (tid < 64) {
    bool all = false;
    for (int it = 0; it < kCutSpin && !all; ++it) {
      const uint32_t f =
          lane < kSampleWgs
              ? __hip_atomic_load(flags + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
              : cut.epoch;
      all = __ballot(f != cut.epoch) == 0ull;
      if (!all) __builtin_amdgcn_s_sleep(4);
    }
    if (tid == 0) s_arr[1] = all ? 1u : 0u;
  }
  __syncthreads();
  if (s_arr[1] == 0u) return;   // the row's waves time out and flag it
  const int64_t row = grp * G + h;
  uint32_t* st = topk::row_at(tws, cut.geom, row).st;
  if (tid == 0) {
    __hip_atomic_store(st + topk::kS_OVER, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (h == 0) __hip_atomic_store(cut.gflag + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The row's keys, read again for each digit with agent-scope loads, in two
  // batches of 16 per thread whose loads are all issued before any is used
  // (the kernel's register count stays the scan's).
  constexpr int kPer = kSampleKeys / kThreads, kBatch = kPer / 2;
  const uint32_t* src = cut.sample + row * (int64_t)topk::kMaxSampleKeys;
  uint32_t* h32 = reinterpret_cast<uint32_t*>(smem);   // the sample's LDS is free now
  const uint32_t tau = topk::radix_cut<kThreads>(
      [&](auto&& f) {
        for (int half = 0; half < 2; ++half) {
          uint32_t key[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u)
            key[u] = __hip_atomic_load(src + (half * kBatch + u) * kThreads + tid,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < kBatch; ++u) f(key[u]);
        }
      },
      (uint32_t)cut.target, h32, h32 + topk::kBins, h32 + topk::kBins + kThreads / 64);
  if (tid == 0) {
    st[topk::kS_TAU] = tau;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the flag clears are out first
    if (cut.publish)
      __hip_atomic_store(st + topk::kS_READY, tau | ready_bits(cut.epoch), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Lane h < G: the ready word of row (group, h); other lanes read as ready.
template <int G>
__device__ __forceinline__ uint32_t cut_word(void* tws, const CutArgs& cut, int64_t grp) {
  const int lane = lane_id();
  if (lane >= G) return ready_bits(cut.epoch);
  uint32_t* p = topk::row_at(tws, cut.geom, grp * G + lane).st + topk::kS_READY;
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The G cuts (as keys and as floats) from the ready words, polled while one
// of this call's is missing; a cut still missing gives NaN (no score is >=
// it) and a key no cut has, and flags its row.
template <int G>
__device__ __forceinline__ void cut_floats(void* tws, const CutArgs& cut, int64_t grp, uint32_t w,
                                           uint32_t (&tk)[G], float (&tf)[G]) {
  const uint32_t rb = ready_bits(cut.epoch);
  for (int it = 0; it < cut.spin && __ballot((w & 0x3FFu) != rb) != 0ull; ++it) {
    __builtin_amdgcn_s_sleep(8);
    w = cut_word<G>(tws, cut, grp);
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)w, h);
    if ((v & 0x3FFu) == rb) {
      tk[h] = v & ~0x3FFu;
      tf[h] = topk::key_float(tk[h]);
    } else {
      tk[h] = 0xFFFFFFFFu;   // low bits set: never a cut
      tf[h] = __builtin_nanf("");
      if (lane_id() == 0)
        atomicOr(&topk::row_at(tws, cut.geom, grp * G + h).st[topk::kS_OVER], 1u);
    }
  }
}

// Candidate emission of the main kernel.  The workgroup's kWaves wave tiles
// (its round of kRoundBlocks blocks) share one region of kWaves * region
// slots per row: every wave counts its scores >= tau per head, the counts are
// prefixed over the waves in LDS, and each wave writes its candidates, as
// (order key, index) in index order, right after those of the waves before
// it, so that the round's candidates lie packed and in index order at the
// front of the region (the selection then copies a round's candidates in one
// piece).  The segment table gets each tile's first slot and count, the
// stamp table the cut the tile used; a round with more candidates than its
// region holds flags the row.
template <int G>
__device__ __forceinline__ void emit_round(const float (&sc)[kNB][G], const uint32_t (&tk)[G],
                                           const float (&tf)[G], int64_t grp, int64_t blk0, int wave,
                                           const topk::RowGeom& geom, void* tws,
                                           uint32_t (*s_ecnt)[G]) {
  const int lane = lane_id();
  const int64_t tile = blk0 / kNB;   // round * kWaves + wave
  const int64_t round = tile / kWaves;
  uint32_t cnt[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    uint32_t c = 0;
#pragma unroll
    for (int b = 0; b < kNB; ++b) c += (uint32_t)__popcll(__ballot(sc[b][h] >= tf[h]));
    cnt[h] = c;
    if (lane == 0) s_ecnt[wave][h] = c;
  }
  __syncthreads();
  const uint32_t idx0 = (uint32_t)(blk0 * kBlock) + (uint32_t)lane;   // this lane's key in block 0
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const topk::RowWs rw = topk::row_at(tws, geom, grp * G + h);
    const uint32_t cap = kWaves * rw.region;
    uint32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t x = s_ecnt[w][h];
      before += w < wave ? x : 0u;
      total += x;
    }
    uint2* dst = reinterpret_cast<uint2*>(rw.cand) + (uint32_t)round * cap;
    const bool fits = before + cnt[h] <= cap;   // uniform: no slot check needed
    uint32_t at = before;
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const bool cand = sc[b][h] >= tf[h];
      const uint64_t mb = __ballot(cand);
      if (mb != 0ull) {
        if (cand) {
          const uint32_t sl = at + __builtin_amdgcn_mbcnt_hi((uint32_t)(mb >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)mb, 0u));
          // Order key without the -0 case: these scores are never -0 (both
          // folds start at +0, and a sum that is exactly 0 rounds to +0).
          const uint32_t u = __float_as_uint(sc[b][h]);
          const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
          if (fits || sl < cap) dst[sl] = make_uint2(key, idx0 + (uint32_t)(b * kBlock));
        }
        at += (uint32_t)__popcll(mb);
      }
    }
    if (lane == 0) {
      rw.seg[2 * tile] = (uint32_t)round * cap + before;
      rw.seg[2 * tile + 1] = cnt[h];
      rw.stamp[2 * tile] = tk[h];
      if (wave == 0 && total > cap) atomicOr(&rw.st[topk::kS_OVER], 1u);
    }
  }
}

// Per-group tables indexed by active slot (the s-th active channel in depth
// order).  Padding slots are never computed; their rows may hold anything.
template <int G>
struct SlotTables {
  float w[kSlots][G];        // q_hj * 2^(11 - t_j)
  float e[kSlots][G];        // fl32(q_hj * (2^-t_j - 1))
};

// ---------------------------------------------------------------------------
// Main kernel: whole rounds, L2 prefetch, scales staged in LDS
// ---------------------------------------------------------------------------

constexpr int kScaleParts = kRoundBlocks / 8;   // 16-byte parts of a slot's round of scales
constexpr int kScalePasses = kD * kScaleParts / kThreads;                            // 2

template <int G>
struct MainShared {
  SlotTables<G> tb;
  alignas(16) float sc[kSlots][kRoundBlocks];      // this round's block scales (a * 2^13;
                                                   // a * 2^-10 in depth-1 slots)
  uint32_t prow[kD * kPlanes];                     // byte offset of every active plane row
  uint8_t sj[kSlots];                              // channel of every active slot
  float qraw[kD][G];                               // the group's queries, by channel
};

struct MainCtx {
  const char* planes;   // the group's plane rows at the tile's first block
  uint32_t pstride;     // bytes between two planes of a channel (nb_store * 8)
  const float* sc;      // this round's staged scales at the wave's first block
  int ob, oh;           // this lane's block and head in the offset fold
};

template <int T, int G>
__device__ __forceinline__ void main_load_plane(const MainCtx& c, int j, int p, ChanLoad<T, G>& L) {
  // Read through the constant address space (the store is read-only while
  // the scan runs): the uniform plane words are then always scalar loads,
  // whatever else the kernel writes.
  typedef const __attribute__((address_space(4))) uint64_t cu64;
  const char* rp = c.planes + (uint32_t)j * (kPlanes * c.pstride) + p * c.pstride;
#pragma unroll
  for (int b = 0; b < kNB; ++b) L.pw[p][b] = *(cu64*)(rp + b * 8);
}

template <int T, int G>
__device__ __forceinline__ void main_load_lds(const MainCtx& c, const SlotTables<G>& tb, int slot,
                                              ChanLoad<T, G>& L) {
  const float* sp = c.sc + slot * kRoundBlocks;
#pragma unroll
  for (int i = 0; i < kNB; ++i) L.A[i] = sp[i];
#pragma unroll
  for (int h = 0; h < G; ++h) L.w[h] = tb.w[slot][h];
  L.e = tb.e[slot][c.oh];
  L.oa = sp[c.ob];
}

template <int T, int G>
__device__ __forceinline__ void main_load(const MainCtx& c, const SlotTables<G>& tb, int slot,
                                          int j, ChanLoad<T, G>& L) {
#pragma unroll
  for (int p = 0; p < T; ++p) main_load_plane<T, G>(c, j, p, L);
  main_load_lds<T, G>(c, tb, slot, L);
}

// The channels of depth T (mask `it`, slots [first, first + cnt)), U at a
// time.  PIPE: two register sets of U channels alternate; the loads of the
// next U slots are issued right after the first instruction of the current
// set (which carries the wait for everything outstanding), so they overlap
// the arithmetic of U channels.  The pipeline reads up to 2U slots past the
// range (padding or other active channels), which are never computed.
template <int T, int G, int U>
struct ChanSet {
  ChanLoad<T, G> ch[U];
};

template <int T, int G, int U>
__device__ __forceinline__ void load_set(const MainCtx& c, const SlotTables<G>& tb, int slot,
                                         ChanIter& it, ChanSet<T, G, U>& S) {
#pragma unroll
  for (int u = 0; u < U; ++u) main_load<T, G>(c, tb, slot + u, it.next(), S.ch[u]);
}

template <int T, int G, int U, class F>
__device__ __forceinline__ void compute_set(const ChanSet<T, G, U>& S, int n, float (&acc)[kNB][G],
                                            float& o, F&& issue_next) {
  compute_chan<T, G>(S.ch[0], acc, o, issue_next);
#pragma unroll
  for (int u = 1; u < U; ++u)
    if (u < n) compute_chan<T, G>(S.ch[u], acc, o, [] {});
}

template <int T, int G, bool PIPE, int U = 1>
__device__ __forceinline__ void main_depth(const MainCtx& c, const SlotTables<G>& tb, int first,
                                           int cnt, ChanIter it, float (&acc)[kNB][G], float& o) {
  if (cnt <= 0) return;
  if (PIPE) {
    ChanSet<T, G, U> A, B;
    load_set<T, G, U>(c, tb, first, it, A);
    int i = 0;
    for (; i + U < cnt; i += 2 * U) {
      compute_set<T, G, U>(A, U, acc, o, [&] { load_set<T, G, U>(c, tb, first + i + U, it, B); });
      compute_set<T, G, U>(B, cnt - i - U, acc, o,
                           [&] { load_set<T, G, U>(c, tb, first + i + 2 * U, it, A); });
    }
    if (i < cnt) compute_set<T, G, U>(A, cnt - i, acc, o, [] {});
  } else {
    for (int i = 0; i < cnt; ++i) {
      ChanLoad<T, G> A;
      main_load<T, G>(c, tb, first + i, it.next(), A);
      compute_chan<T, G>(A, acc, o, [] {});
    }
  }
}

// The vector loads of one round: the block scales of every active slot (kept
// in registers until they are staged) and TOUCHES per plane-row segment of
// the round (kRoundBlocks * 8 = 256 bytes: one 4-byte load per 128-byte
// line), which pull the round's plane lines into L2 ahead of the scalar
// loads.  Thread kScaleParts * s + k loads scales [8k, 8k + 8) of slot s: 16
// aligned bytes when the capacity is a multiple of 8 blocks and the scales
// 16-byte aligned, else eight 2-byte loads.
#ifndef SCAN_TOUCHES
#define SCAN_TOUCHES 2
#endif
constexpr int kTouches = SCAN_TOUCHES;                                  // per row segment
constexpr int kTouchPerThread = kD * kPlanes * kTouches / kThreads;
struct Stage {
  uint4 st[kScalePasses];
  uint32_t sh[kScalePasses][8];   // the same scales, one load each (rows not 16-byte aligned)
  uint32_t tv[kTouchPerThread > 0 ? kTouchPerThread : 1];
};

// Retire a round's L2 touches: their values are folded into `sink`, which
// only keeps the loads alive.
__device__ __forceinline__ void retire_touches(const Stage& S, uint32_t& sink) {
#pragma unroll
  for (int i = 0; i < kTouchPerThread; ++i) sink ^= S.tv[i];
}

// The round's block scales of every active slot: thread kScaleParts * s + k
// loads scales [8k, 8k + 8) of slot s (threads past the active slots load
// channel 0's and ignore them, so every load is issued unconditionally).
template <int G>
__device__ __forceinline__ void issue_scales(const MainShared<G>& sh, int nact,
                                             const char* scales_g, int64_t nb_store, int64_t r0,
                                             bool sv, Stage& S) {
  int tid = threadIdx.x;
  opaque_v(tid);
#pragma unroll
  for (int i = 0; i < kScalePasses; ++i) {
    const int k = tid + i * kThreads;
    const int slot = k / kScaleParts;
    const int64_t ch = slot < nact ? (int64_t)sh.sj[slot] : 0;
    const char* sp = scales_g + (ch * nb_store + r0) * 2 + (k % kScaleParts) * 16;
    if (sv) {
      S.st[i] = *reinterpret_cast<const uint4*>(sp);
    } else {
#pragma unroll
      for (int u = 0; u < 8; ++u) S.sh[i][u] = reinterpret_cast<const uint16_t*>(sp)[u];
    }
  }
}

// The round's L2 touches.  Every load is issued unconditionally (threads
// without a row touch channel 0's first plane row and ignore it), so the
// compiler can count them exactly and the scale wait need not cover them.
template <int G>
__device__ __forceinline__ void issue_touches(const MainShared<G>& sh, int nrows,
                                              const char* planes_g, int64_t r0, Stage& S) {
  int tid = threadIdx.x;
  opaque_v(tid);
#pragma unroll
  for (int i = 0; i < kTouchPerThread; ++i) {
    const int k = tid + i * kThreads;
    const int row = k / kTouches;
    const uint32_t off = row < nrows ? sh.prow[row] : 0u;
    S.tv[i] = *reinterpret_cast<const uint32_t*>(planes_g + off + r0 * 8 +
                                                 (k % kTouches) * (kRoundBlocks * 8 / kTouches));
  }
}

// Write a round's scales to LDS as a * 2^13, a * 2^-10 in the depth-1 slots
// from first1 on (both exact).  The scale loads were
// issued before the L2 touches and vector loads complete in order, so this
// waits for the scales only: the touches stay in flight while the first
// channels are computed.
template <int G>
__device__ __forceinline__ void round_stage(MainShared<G>& sh, int nact, int first1, bool sv,
                                            const Stage& S) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kScalePasses; ++i) {
    const int k = tid + i * kThreads;
    const int slot = k / kScaleParts, part = k % kScaleParts;
    if (slot < nact) {
      uint32_t wd[4] = {S.st[i].x, S.st[i].y, S.st[i].z, S.st[i].w};
      if (!sv) {
#pragma unroll
        for (int u = 0; u < 4; ++u) wd[u] = S.sh[i][2 * u] | (S.sh[i][2 * u + 1] << 16);
      }
      const int ex = slot >= first1 ? -10 : 13;   // depth-1 slots hold a * 2^-10
      float f[8];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        f[2 * u] = __builtin_ldexpf(half_lo(wd[u]), ex);
        f[2 * u + 1] = __builtin_ldexpf(half_lo(wd[u] >> 16), ex);
      }
      float4* dst = reinterpret_cast<float4*>(&sh.sc[slot][part * 8]);
      dst[0] = make_float4(f[0], f[1], f[2], f[3]);
      dst[1] = make_float4(f[4], f[5], f[6], f[7]);
    }
  }
}

// MODE 0: scores only; 1: scores (when `scores` is non-null) and the top-k
// candidates of every wave tile (fathom_scan_topk; needs kRounds == 1);
// 2: as 0, for fathom_scan_topk's second pass over the flagged groups (its
// own instance, so that profiles tell it from full scans).
// `gate` (nullable, per group): a group whose word is 0 is skipped (the
// scan that fathom_scan_topk runs again for rows whose selection failed).
// NR: rounds per workgroup (the second pass takes several, so that its grid,
// launched on every call and empty unless a row failed, is small).
template <int G, int MODE = 0, int NR = kRounds>
__global__ __launch_bounds__(kThreads) void scan_main(
    const uint64_t* __restrict__ planes, const uint16_t* __restrict__ scales, int64_t nb_store,
    const uint8_t* __restrict__ depths, const float* __restrict__ q, int64_t nrounds, int64_t n,
    int64_t wgs_per_group, float* __restrict__ scores, void* tws,
    const uint32_t* __restrict__ gate, CutArgs cut) {
  static_assert(kNB * G <= 64, "one lane per (block, head) in the offset fold");
  static_assert(MODE != 1 || NR == 1, "candidate emission runs one round per workgroup");
  // The sample workgroups' LDS (sample_wg) lives in sh.
  static_assert(sizeof(MainShared<G>) >=
                    kD * kSampleWgBlocks * 2 * 16 + kD * kSampleWgBlocks * 2 + kD * G * 4 + 8,
                "sample scratch");
  static_assert(sizeof(MainShared<G>) >= (topk::kBins + kThreads / 64 + 2) * 4, "cut scratch");
  __shared__ MainShared<G> sh;
  __shared__ float s_o[kWaves][kNB * G];
  __shared__ uint32_t s_ecnt[MODE == 1 ? kWaves : 1][G];   // MODE 1: candidates per wave

  // MODE 1: the first workgroups take the sample and the cuts.
  const uint32_t ncut = MODE == 1 ? sample_workgroups(cut.groups) : 0u;
  if (MODE == 1 && blockIdx.x < ncut) {   // uniform over the workgroup
    sample_wg<G>(cut, blockIdx.x, planes, scales, nb_store, depths, q, tws,
                 reinterpret_cast<char*>(&sh));
    return;
  }
  // XCD-aware remap of the scan's workgroup ids (bijective on [0, nwg)).
  const uint32_t nwg = gridDim.x - ncut;
  const uint32_t per_xcd = nwg / kXcds;
  uint32_t id = blockIdx.x - ncut;
  if (id < per_xcd * kXcds) id = (id % kXcds) * per_xcd + id / kXcds;
  const int64_t grp = id / wgs_per_group;
  if (gate != nullptr && gate[grp] == 0u) return;   // uniform over the workgroup
  const int64_t round0 = (id % wgs_per_group) * NR;
  const int nr = NR > 1 ? (int)min<int64_t>(NR, nrounds - round0) : 1;

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t pstride = (uint32_t)nb_store * 8u;
  const char* planes_g =
      reinterpret_cast<const char*>(planes + grp * kD * (int64_t)kPlanes * nb_store);
  const char* scales_g = reinterpret_cast<const char*>(scales + grp * kD * nb_store);
  // Scale rows as 16-byte vectors, or one 2-byte load per block.
  const bool sv = (nb_store & 7) == 0 && (reinterpret_cast<uintptr_t>(scales) & 15) == 0;
  float* scores_g = scores != nullptr ? scores + grp * G * n : nullptr;

  // The plan's depths and the group's queries are requested together, so they
  // share one round trip to memory (the queries go straight to LDS: held in
  // registers, their loads would be issued only where the plan is known).
  const int dlo = depths[grp * kD + lane_id()], dhi = depths[grp * kD + 64 + lane_id()];
  if (threadIdx.x < kD) {
#pragma unroll
    for (int h = 0; h < G; ++h) sh.qraw[threadIdx.x][h] = q[(grp * G + h) * kD + threadIdx.x];
  }
  const DepthMasks dm = depth_masks(dlo, dhi);
  int cnt[kPlanes];
#pragma unroll
  for (int i = 0; i < kPlanes; ++i) cnt[i] = dm.count[i];
  const int nact = cnt[0] + cnt[1] + cnt[2] + cnt[3];
  const int nrows = 4 * cnt[0] + 3 * cnt[1] + 2 * cnt[2] + cnt[3];

  // Slot tables: waves 0 and 1 own channels 0..127 (thread j, channel j).
  if (tid < 2 * 64) {
    const int j = tid;
    const int t = j < 64 ? dm.tlo : dm.thi;   // depth of channel j, as depth_masks read it
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    if (t > 0) {
      const int di = kPlanes - t;
      int slot = 0, row = 0;
      uint64_t mlo = 0, mhi = 0;   // selected without a dynamic index (no scratch)
#pragma unroll
      for (int i = 0; i < kPlanes; ++i) {
        if (i < di) {
          slot += cnt[i];
          row += cnt[i] * (kPlanes - i);
        }
        if (i == di) {
          mlo = dm.lo[i];
          mhi = dm.hi[i];
        }
      }
      const int rank = (j < 64) ? __popcll(mlo & below) : __popcll(mlo) + __popcll(mhi & below);
      slot += rank;
      row += rank * t;
      const float sw = __builtin_ldexpf(1.0f, 11 - t);
      const float se = __builtin_ldexpf(1.0f, -t) - 1.0f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float qv = sh.qraw[j][h];   // written by this thread
        sh.tb.w[slot][h] = qv * sw;
        sh.tb.e[slot][h] = qv * se;
      }
      sh.sj[slot] = (uint8_t)j;
      for (int p = 0; p < t; ++p) sh.prow[row + p] = ((uint32_t)j * kPlanes + p) * pstride;
    }
  }
  __syncthreads();

  uint32_t sink = 0u;
  Stage S;
  issue_scales<G>(sh, nact, scales_g, nb_store, round0 * kRoundBlocks, sv, S);
  issue_touches<G>(sh, nrows, planes_g, round0 * kRoundBlocks, S);
  const int first1 = cnt[0] + cnt[1] + cnt[2];   // first depth-1 slot
  round_stage<G>(sh, nact, first1, sv, S);
  __syncthreads();

  const bool olane = lane < kNB * G;
  MainCtx c;
  c.pstride = pstride;
  c.ob = olane ? lane / G : 0;
  c.oh = olane ? lane % G : 0;

  for (int r = 0; r < nr; ++r) {
    const int64_t r0 = (round0 + r) * kRoundBlocks;
    if (r + 1 < nr) {
      retire_touches(S, sink);
      issue_scales<G>(sh, nact, scales_g, nb_store, r0 + kRoundBlocks, sv, S);
      issue_touches<G>(sh, nrows, planes_g, r0 + kRoundBlocks, S);
    }

    DepthMasks rm = dm;   // per-round copy: nothing derived from it is hoisted
#pragma unroll
    for (int i = 0; i < kPlanes; ++i) {
      opaque_s(rm.lo[i]);
      opaque_s(rm.hi[i]);
      opaque_s(rm.count[i]);
    }
    const int64_t blk0 = r0 + wave * kNB;
    c.planes = planes_g + blk0 * 8;
    c.sc = &sh.sc[0][wave * kNB];
    float acc[kNB][G];
#pragma unroll
    for (int b = 0; b < kNB; ++b)
#pragma unroll
      for (int h = 0; h < G; ++h) acc[b][h] = 0.0f;
    float o = 0.0f;
    const int* rc = rm.count;
    main_depth<4, G, false>(c, sh.tb, 0, rc[0], ChanIter{rm.lo[0], rm.hi[0]}, acc, o);
    main_depth<3, G, false>(c, sh.tb, rc[0], rc[1], ChanIter{rm.lo[1], rm.hi[1]}, acc, o);
    // One round per workgroup: the touches have landed by now.  Retiring them
    // here (the empty asm keeps the compiler from sinking the XORs to the end)
    // frees their registers for the pipelined depths below: 78 at G = 4,
    // which fits 6 waves per SIMD instead of 5.
    if (NR == 1) {
      retire_touches(S, sink);
      asm volatile("" : "+v"(sink));
    }
    main_depth<2, G, true>(c, sh.tb, rc[0] + rc[1], rc[2], ChanIter{rm.lo[2], rm.hi[2]}, acc, o);
    // MODE 1: the ready words of the group's cuts, read here so that they
    // have arrived (and the cuts are out) by the time the tile is emitted.
    uint32_t cw = 1u;
    if (MODE == 1) cw = cut_word<G>(tws, cut, grp);
    main_depth<1, G, true, SCAN_U1>(c, sh.tb, rc[0] + rc[1] + rc[2], rc[3],
                                    ChanIter{rm.lo[3], rm.hi[3]}, acc, o);
    finish_tile<G>(acc, o, kNB - 1, n, scores_g != nullptr ? scores_g + blk0 * kBlock : nullptr,
                   s_o[wave]);
    if (MODE == 1) {
      uint32_t tk[G];
      float tf[G];
      cut_floats<G>(tws, cut, grp, cw, tk, tf);
      emit_round<G>(acc, tk, tf, grp, blk0, wave, cut.geom, tws, s_ecnt);
    }

    if (r + 1 < nr) {
      __syncthreads();   // every wave is done with this round's scales
      round_stage<G>(sh, nact, first1, sv, S);
      __syncthreads();
    }
  }
  if (NR > 1) retire_touches(S, sink);
  asm volatile("" ::"v"(sink));   // keeps the L2 touches alive
}

// ---------------------------------------------------------------------------
// Tail kernel: the wave tiles from first_blk on (the blocks after the last
// whole round; every block of a group whose plane array needs 64-bit
// offsets), one workgroup per tile, one wave per block, lane i = token i.
// ---------------------------------------------------------------------------
//
// The tile's plane rows with p < t_j and its scales are staged in LDS (one
// round of loads after the depths; blocks past the row's end read the last
// block, and rows past a channel's depth are not loaded), then every lane
// folds its own token in the stated order: depths 4 to 1, ascending j,
//   U_h = fma(w_hj, m_j, U_h),  o_h = fma(e_hj, a_j, o_h),  S_h = U_h + o_h,
// with m_j = c'_j * (a_j * 2^-10) (exact: a 4-bit by 11-bit product), the
// same values the main kernel folds per block.  8- and 2-byte loads only,
// so any capacity and alignment the arguments allow.
constexpr int kTailThreads = kNB * 64;   // one wave per block of the tile
static_assert(kTailThreads == kD * kPlanes, "one thread per plane row of the tile");

// MODE and `gate` as in scan_main (with MODE 1 the tail's tiles, the last one
// possibly partial, emit their candidates).
template <int G, int MODE = 0>
__global__ __launch_bounds__(kTailThreads) void scan_tail(
    const uint64_t* __restrict__ planes, const uint16_t* __restrict__ scales, int64_t nb_store,
    const uint8_t* __restrict__ depths, const float* __restrict__ q, int64_t first_blk,
    int64_t nblk, int64_t n, float* __restrict__ scores, void* tws,
    const uint32_t* __restrict__ gate) {
  __shared__ uint64_t s_w[kD * kPlanes][kNB];   // row (channel, plane), block of the tile
  __shared__ uint16_t s_sc[kD][kNB];
  __shared__ float s_q[G][kD];
  __shared__ uint32_t s_cnt[G][kNB];
  const int64_t grp = blockIdx.y;
  if (gate != nullptr && gate[grp] == 0u) return;   // uniform over the workgroup
  const int tid = threadIdx.x, lane = lane_id();
  const int b = __builtin_amdgcn_readfirstlane(tid >> 6);   // this wave's block
  const int64_t blk0 = first_blk + (int64_t)blockIdx.x * kNB;
  const int last = (int)min<int64_t>(kNB, nblk - blk0) - 1;  // last block of the tile in the row
  const uint8_t* dg = depths + grp * kD;
  const uint64_t* pg = planes + grp * kD * (int64_t)kPlanes * nb_store + blk0;
  const uint16_t* sg = scales + grp * kD * nb_store + blk0;
  // Thread r stages plane row r = (channel r / 4, plane r % 4); threads below
  // kD also the scale row and the queries of channel tid.
  const int tr = min((int)dg[tid >> 2], kPlanes);
  const int tl0 = min((int)dg[lane], kPlanes), tl1 = min((int)dg[64 + lane], kPlanes);
  if (tid < kD) {
#pragma unroll
    for (int u = 0; u < kNB; ++u) s_sc[tid][u] = sg[(int64_t)tid * nb_store + min(u, last)];
#pragma unroll
    for (int h = 0; h < G; ++h) s_q[h][tid] = q[(grp * G + h) * kD + tid];
  }
  if ((tid & (kPlanes - 1)) < tr) {
    const uint64_t* rp = pg + (int64_t)tid * nb_store;
#pragma unroll
    for (int u = 0; u < kNB; ++u) s_w[tid][u] = rp[min(u, last)];
  }
  __syncthreads();

  float U[G], o[G];
#pragma unroll
  for (int h = 0; h < G; ++h) U[h] = o[h] = 0.0f;
  const int hsel = lane >> 5, bit = lane & 31;
#pragma unroll
  for (int t = kPlanes; t >= 1; --t) {
    // The channels of depth t, ascending.
    ChanIter it{__ballot(tl0 == t), __ballot(tl1 == t)};
    const int cnt = __popcll(it.lo) + __popcll(it.hi);
    const float sw = __builtin_ldexpf(1.0f, 11 - t), se = __builtin_ldexpf(1.0f, -t) - 1.0f;
    for (int i = 0; i < cnt; ++i) {
      const int j = it.next();
      const uint32_t* wp = reinterpret_cast<const uint32_t*>(&s_w[j * kPlanes][b]) + hsel;
      uint32_t cp = 0u;
      for (int p = 0; p < t; ++p) cp = 2 * cp + ((wp[p * 2 * kNB] >> bit) & 1u);
      const float a = half_lo(s_sc[j][b]);
      const float m = (float)cp * __builtin_ldexpf(a, -10);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float qv = s_q[h][j];
        U[h] = __builtin_fmaf(qv * sw, m, U[h]);
        o[h] = __builtin_fmaf(qv * se, a, o[h]);
      }
    }
  }
  float S[G];
#pragma unroll
  for (int h = 0; h < G; ++h) S[h] = U[h] + o[h];
  if (scores != nullptr && b <= last) {
#pragma unroll
    for (int h = 0; h < G; ++h) scores[(grp * G + h) * n + (blk0 + b) * kBlock + lane] = S[h];
  }
  if (MODE == 1) {
    // The tile's candidates in index order: per head, block b's count of
    // scores >= tau, prefixed over the blocks in LDS.
    const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int64_t tile = blk0 / kNB;
    bool cand[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const topk::RowWs rw = topk::row_ws(tws, n, kTileKeys, grp * G + h);
      cand[h] = b <= last && S[h] >= topk::key_float(rw.st[topk::kS_TAU]);
      const uint64_t mk = __ballot(cand[h]);
      if (lane == 0) s_cnt[h][b] = (uint32_t)__popcll(mk);
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const topk::RowWs rw = topk::row_ws(tws, n, kTileKeys, grp * G + h);
      const uint32_t base = (uint32_t)tile * rw.region;
      uint32_t before = 0, total = 0;
#pragma unroll
      for (int u = 0; u < kNB; ++u) {
        const uint32_t c = s_cnt[h][u];
        before += u < b ? c : 0u;
        total += c;
      }
      const uint64_t mk = __ballot(cand[h]);
      const uint32_t sl = before + (uint32_t)__popcll(mk & below);
      if (cand[h] && sl < rw.region)
        reinterpret_cast<uint2*>(rw.cand)[base + sl] =
            make_uint2(topk::order_key(S[h]), (uint32_t)((blk0 + b) * kBlock + lane));
      if (tid == 0) {
        rw.seg[2 * tile] = base;
        rw.seg[2 * tile + 1] = total;
        rw.stamp[2 * tile] = rw.st[topk::kS_TAU];
        if (total > rw.region) atomicOr(&rw.st[topk::kS_OVER], 1u);
      }
    }
  }
}

// With timing events, the first launch records ev_start and the last one
// ev_stop from the kernels' own dispatch timestamps (no marker packets).
template <int G>
void launch_scan_g(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                   const uint8_t* depths, const float* q, int64_t groups, int64_t n,
                   float* scores, hipStream_t stream, hipEvent_t ev_start = nullptr,
                   hipEvent_t ev_stop = nullptr) {
  const int64_t nblk = n / kBlock;
  // Main kernel: 32-bit offsets into a group's plane array.
  const bool fast = nb_store <= kMaxFastBlocks;
  const int64_t nrounds = fast ? nblk / kRoundBlocks : 0;
  const int64_t first = nrounds * kRoundBlocks;
  const bool timed = ev_start != nullptr || ev_stop != nullptr;
  if (nrounds > 0) {
    const int64_t wgs = (nrounds + kRounds - 1) / kRounds;
    const dim3 grid((unsigned)(wgs * groups)), block(kThreads);
    if (timed)
      hipExtLaunchKernelGGL((scan_main<G, 0>), grid, block, 0, stream, ev_start,
                            first < nblk ? nullptr : ev_stop, 0u, planes, scales, nb_store,
                            depths, q, nrounds, n, wgs, scores, (void*)nullptr,
                            (const uint32_t*)nullptr, CutArgs{});
    else
      hipLaunchKernelGGL((scan_main<G, 0>), grid, block, 0, stream, planes, scales, nb_store,
                         depths, q, nrounds, n, wgs, scores, (void*)nullptr,
                         (const uint32_t*)nullptr, CutArgs{});
  }
  if (first < nblk) {
    const dim3 grid((unsigned)((nblk - first + kNB - 1) / kNB), (unsigned)groups),
        block(kTailThreads);
    if (timed)
      hipExtLaunchKernelGGL((scan_tail<G, 0>), grid, block, 0, stream,
                            nrounds > 0 ? nullptr : ev_start, ev_stop, 0u, planes, scales,
                            nb_store, depths, q, first, nblk, n, scores, (void*)nullptr,
                            (const uint32_t*)nullptr);
    else
      hipLaunchKernelGGL((scan_tail<G, 0>), grid, block, 0, stream, planes, scales, nb_store,
                         depths, q, first, nblk, n, scores, (void*)nullptr,
                         (const uint32_t*)nullptr);
  }
}

}  // namespace

// fathom_scan_topk.  Fused path (64k to 2M keys, 32-bit offsets into a
// group's plane array): sample -> cut per row -> scan that writes the scores
// (when a buffer is given) and every score >= tau into its wave tile's
// candidate region (whole rounds in the main kernel, the blocks after the
// last whole round in the tail kernel) -> selection from the candidates.
// Without a score buffer, rows whose candidates cannot give the selection
// (fewer than k, or a region overflowed) are flagged: their groups are
// scanned again into the workspace's score area and selected from there; the
// other groups' work ends at once.  Otherwise the two calls run as they are.
// fathom_test_cut_hooks' settings.
static std::atomic<int> g_cut_publish{1}, g_cut_spin{kCutSpin};

template <int G>
hipError_t launch_scan_topk_g(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                              const uint8_t* depths, const float* q, int64_t groups, int64_t n,
                              int k, float* scores, int32_t* indices, void* ws,
                              hipStream_t stream) {
  const int64_t rows = groups * G, R = kTileKeys;
  const int64_t nblk = n / kBlock, nrounds = nblk / kRoundBlocks, first = nrounds * kRoundBlocks;
  const topk::FusedWs fw = topk::fused_ws(ws, rows, groups, n, R);
  float* sc = scores != nullptr ? scores : fw.scores;
  const bool fused = kRounds == 1 && n >= kFusedMinKeys && topk::n_chunks(n, R) <= kFusedMaxTiles &&
                     nb_store <= kMaxFastBlocks;
  if (!fused) {   // the two calls one after the other
    launch_scan_g<G>(planes, scales, nb_store, depths, q, groups, n, sc, stream);
    return launch_topk(sc, rows, n, k, indices, ws, stream);
  }
  const int64_t ntiles = nblk / kNB, rstride = ntiles / kSampleRuns;   // >= 16 tiles
  // The call's epoch tells its sample flags and published cuts from those of
  // earlier calls.
  static std::atomic<uint32_t> epochs{0};
  uint32_t epoch = ++epochs;
  if (epoch == 0u) epoch = ++epochs;   // 0: zeroed memory is never taken for this call
  // The cut leaves about 1.6x the sample's share of k (plus 16 sampled keys)
  // at or above it, so that fewer than k candidates is rare.
  const double share = (double)k * (double)kSampleKeys / (double)n;
  const int target = (int)std::min<double>((double)kSampleKeys, std::ceil(1.6 * share + 16.0));
  // The scan (MODE 1: with candidates, the sample and the cuts taken by its
  // first workgroups; MODE 2, gated: the second pass).
  auto scan = [&](auto mode, float* out, const uint32_t* gate) {
    constexpr int M = decltype(mode)::value;
    constexpr int NR = M == 2 ? kRescanRounds : 1;
    void* tws = M == 1 ? fw.rows : nullptr;
    const CutArgs cut = M == 1 ? CutArgs{fw.sample, target, (int)groups, topk::row_geom(n, R),
                                         g_cut_publish.load(), g_cut_spin.load(), rstride,
                                         fw.gflag, fw.sflag, epoch}
                               : CutArgs{};
    const int64_t wgs = (nrounds + NR - 1) / NR;
    const unsigned grid =
        (unsigned)(wgs * groups) + (M == 1 ? sample_workgroups((int)groups) : 0u);
    hipLaunchKernelGGL((scan_main<G, M, NR>), dim3(grid), dim3(kThreads), 0, stream, planes,
                       scales, nb_store, depths, q, nrounds, n, wgs, out, tws, gate, cut);
    if (first < nblk)
      hipLaunchKernelGGL((scan_tail<G, M>), dim3((unsigned)((nblk - first + kNB - 1) / kNB),
                                                 (unsigned)groups),
                         dim3(kTailThreads), 0, stream, planes, scales, nb_store, depths, q, first,
                         nblk, n, out, tws, gate);
  };
  scan(std::integral_constant<int, 1>(), scores, nullptr);
  // The main kernel packs each round's kWaves tiles (emit_round).
  const int64_t npacked = kWaves * nrounds;
  hipError_t e = launch_fused_resolve(scores, rows, n, R, k, indices, fw.rows, 0, fw.gflag, G,
                                      kWaves, npacked, stream);
  if (e != hipSuccess || scores != nullptr) return e;
  scan(std::integral_constant<int, 2>(), fw.scores, fw.gflag);
  return launch_fused_resolve(fw.scores, rows, n, R, k, indices, fw.rows, 1, fw.gflag, G, kWaves,
                              npacked, stream);
}

void set_cut_hooks(int publish, int spin_limit) {
  g_cut_publish.store(publish);
  g_cut_spin.store(spin_limit);
}

int64_t scan_max_workgroups(int64_t groups, int64_t n) {
  const int64_t nblk = n / kBlock;
  return groups * ((nblk + kRoundBlocks - 1) / kRoundBlocks);
}

hipError_t launch_scan(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                       const uint8_t* depths, const float* q, int64_t groups, int G, int64_t n,
                       float* scores, hipStream_t stream, hipEvent_t ev_start,
                       hipEvent_t ev_stop) {
  switch (G) {
    case 1:
      launch_scan_g<1>(planes, scales, nb_store, depths, q, groups, n, scores, stream, ev_start,
                        ev_stop);
      break;
    case 2:
      launch_scan_g<2>(planes, scales, nb_store, depths, q, groups, n, scores, stream, ev_start,
                        ev_stop);
      break;
    case 3:
      launch_scan_g<3>(planes, scales, nb_store, depths, q, groups, n, scores, stream, ev_start,
                        ev_stop);
      break;
    case 4:
      launch_scan_g<4>(planes, scales, nb_store, depths, q, groups, n, scores, stream, ev_start,
                        ev_stop);
      break;
    case 5:
      launch_scan_g<5>(planes, scales, nb_store, depths, q, groups, n, scores, stream, ev_start,
                        ev_stop);
      break;
    case 6:
      launch_scan_g<6>(planes, scales, nb_store, depths, q, groups, n, scores, stream, ev_start,
                        ev_stop);
      break;
    case 7:
      launch_scan_g<7>(planes, scales, nb_store, depths, q, groups, n, scores, stream, ev_start,
                        ev_stop);
      break;
    case 8:
      launch_scan_g<8>(planes, scales, nb_store, depths, q, groups, n, scores, stream, ev_start,
                        ev_stop);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t scan_topk_workspace_bytes(int64_t groups, int G, int64_t n, int k) {
  const int64_t rows = groups * G;
  (void)k;
  return topk::fused_front_bytes(rows, groups, n, kTileKeys) +
         topk::align256((size_t)rows * n * sizeof(float));
}

hipError_t launch_scan_topk(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                            const uint8_t* depths, const float* q, int64_t groups, int G,
                            int64_t n, int k, float* scores, int32_t* indices, void* ws,
                            hipStream_t stream) {
  switch (G) {
#define FATHOM_SCAN_TOPK_CASE(g)                                                                 \
  case g:                                                                                        \
    return launch_scan_topk_g<g>(planes, scales, nb_store, depths, q, groups, n, k, scores,     \
                                 indices, ws, stream);
    FATHOM_SCAN_TOPK_CASE(1)
    FATHOM_SCAN_TOPK_CASE(2)
    FATHOM_SCAN_TOPK_CASE(3)
    FATHOM_SCAN_TOPK_CASE(4)
    FATHOM_SCAN_TOPK_CASE(5)
    FATHOM_SCAN_TOPK_CASE(6)
    FATHOM_SCAN_TOPK_CASE(7)
    FATHOM_SCAN_TOPK_CASE(8)
#undef FATHOM_SCAN_TOPK_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fathom
