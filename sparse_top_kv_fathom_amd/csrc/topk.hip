// fathom_topk on gfx950: exact per-row top-k of fp32 scores.
//
// "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches",
// §2: the keys kept for attention are the top-k under the method's scores,
// chosen per query head.  Selection order: score descending, lower index
// first on equal scores; the k indices of a row are returned ascending.
//
// Scores map to order-preserving 32-bit keys (fp32 bits with the sign
// folded, -0 mapped to +0).  Per row:
//   cut     — one workgroup per row takes 16 runs of 1024 keys spread over
//             the row (the whole row when it is short) and places a cut tau
//             that leaves, by that sample, comfortably more than k keys at or
//             above it (two radix digits over the sampled keys); clears the
//             row's overflow flag;
//   compact — one pass over the row writes every key >= tau (key, index) of
//             a chunk, in index order, to that chunk's own region of the
//             row's candidate buffer, and its count;
//   resolve — one workgroup per row: prefixes the chunk counts, loads the
//             candidates into registers (each wave a contiguous segment of
//             them in index order), finds the k-th largest key T with two
//             radix digits counted from tau and the keys == T still needed,
//             and writes every selected index (every key > T, the earliest
//             keys == T) at its place, so the row comes out in index order
//             without a sort.
// If the cut fails (fewer than k keys >= tau, or a chunk with more than its
// region holds: heavy ties or adversarial rows), or there are more candidates
// than the registers hold, the resolve workgroup does all of it alone, from
// the scores or the regions: same result, many more passes.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "fathom_internal.h"
#include "topk_layout.h"
#include "topk_select.h"

namespace fathom {

// Fixed scratch of fathom_topk_noalloc: the selection's workspace for callers
// that cannot allocate.  One copy per GPU the library runs on, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever passed to a kernel.
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

using namespace topk;

constexpr int kThreads = 256;
constexpr int kWavesPerWg = kThreads / 64;
constexpr int kPerThread = 32;                       // keys per thread in a chunk
constexpr int kChunk = kThreads * kPerThread;        // 8192 keys per workgroup chunk
static_assert(kChunk == kCompactChunk, "compaction regions are whole chunks");
constexpr int kWaveKeys = 64 * kPerThread;           // 2048 contiguous keys per wave
constexpr int kResolveThreads = 1024;
constexpr int kGroups = 4096;                        // chunk groups of the one-workgroup write

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// The scores of one chunk in registers: wave w of the workgroup owns keys
// [w * 2048, w * 2048 + 2048) of the chunk; lane l holds, for i = 0..7, the 4
// keys at wave offset (i * 64 + l) * 4.
struct ChunkVals {
  float v[kPerThread / 4][4];
};

// Offset of the key (i, c) of this thread from the chunk's first key.
// Offsets and indices within a row fit in 32 bits (rows have fewer than 2^31
// keys), so a load takes the chunk's (uniform) first key plus one 32-bit
// offset.
__device__ __forceinline__ uint32_t key_off(int i, int c) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  return (uint32_t)(wave * kWaveKeys + (i * 64 + lane) * 4 + c);
}

__device__ __forceinline__ bool chunk_full(const float* src, int64_t n, int64_t c0) {
  return (reinterpret_cast<uintptr_t>(src) & 15) == 0 && c0 + kChunk <= n;
}

// FULL: the chunk lies inside the row and the row start is 16-byte aligned,
// so every key is valid and the loads are 16-byte vectors.
// Padding of a partial chunk reads NaN, never >= a cut: no key past the row
// is a candidate.
template <bool FULL>
__device__ __forceinline__ void load_vals(const float* __restrict__ src, int64_t n, int64_t c0,
                                          ChunkVals& V) {
  const float* __restrict__ base = src + c0;
  if (FULL) {
    typedef float f4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < kPerThread / 4; ++i) {
      const f4 x = __builtin_nontemporal_load(reinterpret_cast<const f4*>(base + key_off(i, 0)));
      V.v[i][0] = x.x;
      V.v[i][1] = x.y;
      V.v[i][2] = x.z;
      V.v[i][3] = x.w;
    }
  } else {
    const uint32_t lim = (uint32_t)min<int64_t>(n - c0, kChunk);   // keys of the chunk in the row
#pragma unroll
    for (int i = 0; i < kPerThread / 4; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t o = key_off(i, c);
        V.v[i][c] = o < lim ? base[o] : __builtin_nanf("");
      }
    }
  }
}

// Exclusive prefix of cnt[0, m) in place, over the workgroup (m <= kGroups).
template <int NT>
__device__ __forceinline__ void block_prefix_inplace(uint32_t* cnt, int m, uint32_t* s_tmp) {
  const int per = (m + NT - 1) / NT;
  const int g0 = min(m, (int)threadIdx.x * per), g1 = min(m, g0 + per);
  uint32_t sum = 0;
  for (int g = g0; g < g1; ++g) sum += cnt[g];
  uint32_t tot;
  uint32_t run = block_exclusive_sum<NT>(sum, s_tmp, tot);
  for (int g = g0; g < g1; ++g) {
    const uint32_t v = cnt[g];
    cnt[g] = run;
    run += v;
  }
}

// The cut and the compaction in one launch.  Its first `rows` workgroups
// take one row's cut each from a sample of the row: 8 runs of 1024 keys
// spread evenly over the row (the whole row when it has at most 8192 keys),
// 32 per thread; tau = radix_cut of them at the target-th largest, target =
// the sample's share of k raised by 60% plus 16 keys (k itself for a whole
// row, where the cut then lies at or just below the k-th key).  tau goes to
// the row's state for the selection and is published in the row's ready word
// as tau | epoch << 1 | 1 (tau's low 10 bits are clear) with an agent-scope
// atomic store.  The other workgroups each compact chunks (see compact_chunk):
// they load their chunk, then read the ready word (agent-scope loads) until
// it carries this call's epoch, polling a bounded number of times.  A chunk
// whose cut never came writes no candidates and stamps an impossible cut, and
// the selection checks every chunk's stamp against the row's cut, so no
// timing or stale word can change a result: it can only send a row to the
// selection from its scores.
constexpr int kCutRuns = 8, kCutRun = 1024, kCutKeys = kCutRuns * kCutRun;
constexpr int kCutPer = kCutKeys / kThreads;
static_assert(kCutPer == 32, "32 sampled keys per thread");
constexpr size_t kCutHistBytes = kBins * sizeof(uint32_t);
constexpr int kTopkCutSpin = 2048;              // polls (about 0.2 us each) of a cut not yet out
constexpr int64_t kMaxCompactWgs = 1 << 22;     // compaction workgroups at most (then they loop)
constexpr uint32_t kNoCut = 0xFFFFFFFFu;        // a stamp no cut equals (a cut's low bits are 0)

__device__ __forceinline__ uint32_t cut_ready_bits(uint32_t epoch) {
  return ((epoch & 0x1FFu) << 1) | 1u;
}

struct TopkCut {
  uint32_t epoch;   // the call's epoch (its low 9 bits are used)
  int publish;      // 1; 0 only under fathom_test_cut_hooks
  int spin;         // the poll limit
};

__device__ __forceinline__ void cut_row(const float* __restrict__ src, int64_t n, int k,
                                        const RowWs& r, const TopkCut& cut, uint32_t* s_hist,
                                        uint32_t* s_tmp, uint32_t* s_sel) {
  const int tid = threadIdx.x;
  const bool whole = n <= (int64_t)kCutKeys;
  const int nkeys = whole ? (int)n : kCutKeys;
  uint32_t key[kCutPer];
  if (whole) {
#pragma unroll
    for (int u = 0; u < kCutPer; ++u) {
      const int64_t i = tid + (int64_t)u * kThreads;
      key[u] = i < n ? order_key(src[i]) : 0u;
    }
  } else {
    // Run c = tid / 32 starts at c * (n - 1024) / 7 (rounded down to 4 keys);
    // thread t takes its keys [32 (t mod 32), 32 (t mod 32) + 32).
    const int64_t start = ((tid >> 5) * ((n - kCutRun) / (kCutRuns - 1))) & ~(int64_t)3;
    const float* p = src + start + (tid & 31) * kCutPer;
    if ((reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      typedef float f4 __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int u = 0; u < kCutPer / 4; ++u) {
        const f4 x = *reinterpret_cast<const f4*>(p + 4 * u);
        key[4 * u] = order_key(x.x);
        key[4 * u + 1] = order_key(x.y);
        key[4 * u + 2] = order_key(x.z);
        key[4 * u + 3] = order_key(x.w);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kCutPer; ++u) key[u] = order_key(p[u]);
    }
  }
  uint32_t need = (uint32_t)k;
  if (!whole) {
    const double share = (double)k * (double)nkeys / (double)n;
    need = (uint32_t)min<double>((double)nkeys, ceil(1.6 * share + 16.0));
  }
  // Only a whole-row sample has slots past the row's end to skip.
  const uint32_t tau = radix_cut<kThreads>(
      [&](auto&& f) {
#pragma unroll
        for (int u = 0; u < kCutPer; ++u)
          if (!whole || tid + (int64_t)u * kThreads < n) f(key[u]);
      },
      need, s_hist, s_tmp, s_sel);
  if (tid == 0) {
    r.st[kS_TAU] = tau;
    if (cut.publish)
      __hip_atomic_store(&r.st[kS_READY], tau | cut_ready_bits(cut.epoch), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Every key >= tau of chunk `chunk` (keys [c0, c0 + kChunk) of the row)
// written in index order to the chunk's region of the candidate buffer; the
// count and the cut used go to the segment and stamp tables (a count above
// the region sends the row to the slow path).  The test is a float compare
// against the cut (a NaN, the padding included, is never a candidate); order
// keys are formed for candidates only.
template <bool F>
__device__ __forceinline__ void compact_chunk(const float* __restrict__ src, int64_t n, int64_t c0,
                                              int64_t chunk, const RowWs& r, const TopkCut& cut,
                                              uint32_t* s_cnt, uint32_t* s_cut) {
  const int wave = threadIdx.x >> 6;
  ChunkVals V;
  load_vals<F>(src, n, c0, V);
  if (threadIdx.x == 0) {
    const uint32_t rb = cut_ready_bits(cut.epoch);
    uint32_t w = __hip_atomic_load(&r.st[kS_READY], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int it = 0; it < cut.spin && (w & 0x3FFu) != rb; ++it) {
      __builtin_amdgcn_s_sleep(8);
      w = __hip_atomic_load(&r.st[kS_READY], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    *s_cut = (w & 0x3FFu) == rb ? (w & ~0x3FFu) : kNoCut;
  }
  __syncthreads();
  const uint32_t tau = *s_cut;
  const uint32_t base = (uint32_t)chunk * r.region;
  if (tau == kNoCut) {   // uniform: the cut never came
    if (threadIdx.x == 0) {
      r.seg[2 * chunk] = base;
      r.seg[2 * chunk + 1] = 0u;
      r.stamp[2 * chunk] = kNoCut;
    }
    return;
  }
  const float tauf = key_float(tau);
  uint32_t ncand = 0;
#pragma unroll
  for (int i = 0; i < kPerThread / 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      ncand += (uint32_t)__popcll(__ballot(V.v[i][c] >= tauf));
  if (lane_id() == 0) s_cnt[wave] = ncand;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerWg; ++w) t += s_cnt[w];
    r.seg[2 * chunk] = base;
    r.seg[2 * chunk + 1] = t;
    r.stamp[2 * chunk] = tau;
  }
  if (ncand != 0u) {
    // Slots follow index order: the keys of step i are (lane, c) with index
    // ascending in lane, then c.
    uint32_t slot = 0;
    for (int w = 0; w < wave; ++w) slot += s_cnt[w];
    const uint64_t below = lanes_below();
#pragma unroll
    for (int i = 0; i < kPerThread / 4; ++i) {
      bool cand[4];
      uint64_t m[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        cand[c] = V.v[i][c] >= tauf;
        m[c] = __ballot(cand[c]);
      }
      if ((m[0] | m[1] | m[2] | m[3]) == 0ull) continue;
      uint32_t sl = slot;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sl += (uint32_t)__popcll(m[c] & below);
        slot += (uint32_t)__popcll(m[c]);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (cand[c]) {
          if (sl < r.region)
            reinterpret_cast<uint2*>(r.cand)[base + sl] =
                make_uint2(order_key(V.v[i][c]), (uint32_t)c0 + key_off(i, c));
          ++sl;
        }
      }
    }
  }
}

// Workgroups [0, rows): the rows' cuts; the others: chunks w, w + nwg, ...
// of the rows' chunks in row-major order (nwg compaction workgroups).
__global__ __launch_bounds__(kThreads) void topk_cut_compact(const float* __restrict__ scores,
                                                             int64_t rows, int64_t n, int k,
                                                             void* ws, int64_t nwg,
                                                             TopkCut cut) {
  // The cut's counts in dynamic LDS (kCutHistBytes at launch): a static
  // array would make the compiler size the compaction's registers for the
  // occupancy that array allows, which is lower than the registers allow.
  extern __shared__ uint32_t s_hist[];
  __shared__ uint32_t s_tmp[kWavesPerWg];
  __shared__ uint32_t s_sel[2];
  __shared__ uint32_t s_cnt[kWavesPerWg];
  __shared__ uint32_t s_cut;
  const int64_t id = blockIdx.x;
  if (id < rows) {
    const RowWs r = row_ws(ws, n, kChunk, id);
    cut_row(scores + id * n, n, k, r, cut, s_hist, s_tmp, s_sel);
    return;
  }
  const int64_t nc = n_chunks(n, kChunk);
  for (int64_t g = id - rows; g < rows * nc; g += nwg) {
    if (g != id - rows) __syncthreads();   // s_cnt and s_cut of the last chunk are read
    const int64_t row = g / nc, chunk = g - row * nc;
    const RowWs r = row_ws(ws, n, kChunk, row);
    const int64_t c0 = chunk * kChunk;
    const float* src = scores + row * n;
    if (chunk_full(src, n, c0)) compact_chunk<true>(src, n, c0, chunk, r, cut, s_cnt, &s_cut);
    else compact_chunk<false>(src, n, c0, chunk, r, cut, s_cnt, &s_cut);
  }
}

// The keys the one-workgroup path selects among: the candidate regions, or
// (direct mode) the row itself.
struct ResolveSrc {
  const uint2* cand;      // (key, index) pairs; chunk c's at seg[2c], seg[2c + 1] of them
  const uint32_t* seg;
  const float* scores;
  int64_t n, nc, R;       // keys, regions and keys per region of the row
  uint32_t region;
  bool direct;
};

// f(key, index) for every key, spread over the workgroup, in any order;
// four loads in flight per thread.
template <class F>
__device__ __forceinline__ void for_each_key(const ResolveSrc s, F&& f) {
  constexpr int kU = 4;
  if (!s.direct) {
    // Wave w takes chunks w, w + 16, ..., 64 candidates at a time.
    const int wave = threadIdx.x >> 6, lane = lane_id();
    for (int64_t c = wave; c < s.nc; c += kResolveThreads / 64) {
      const uint32_t b = s.seg[2 * c], cnt = s.seg[2 * c + 1];
      for (uint32_t o0 = lane; o0 < cnt; o0 += kU * 64) {
        uint2 e[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const uint32_t o = o0 + u * 64;
          e[u] = o < cnt ? s.cand[b + o] : make_uint2(0u, 0u);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (o0 + u * 64 < cnt) f(e[u].x, e[u].y);
      }
    }
  } else {
    for (int64_t i0 = threadIdx.x; i0 < s.n; i0 += kU * kResolveThreads) {
      float v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = i0 + u * kResolveThreads;
        v[u] = i < s.n ? s.scores[i] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t i = i0 + u * kResolveThreads;
        if (i < s.n) f(order_key(v[u]), (uint32_t)i);
      }
    }
  }
}

// One wave visits the keys of chunks [cb, ce) in index order, 64 at a time:
// g(key, index, valid) with every lane of the wave taking part.
template <class G>
__device__ __forceinline__ void walk_chunks(const ResolveSrc s, int64_t cb, int64_t ce, G&& g) {
  const int lane = lane_id();
  for (int64_t c = cb; c < ce; ++c) {
    if (!s.direct) {
      const uint32_t s0 = s.seg[2 * c], cnt = s.seg[2 * c + 1];
      for (uint32_t o = 0; o < cnt; o += 64) {
        const bool v = o + lane < cnt;
        const uint2 e = v ? s.cand[s0 + o + lane] : make_uint2(0u, 0u);
        g(e.x, e.y, v);
      }
    } else {
      const int64_t e = min<int64_t>(s.n, (c + 1) * s.R);
      for (int64_t i0 = c * s.R; i0 < e; i0 += 64) {
        const int64_t i = i0 + lane;
        const bool v = i < e;
        g(v ? order_key(s.scores[i]) : 0u, (uint32_t)i, v);
      }
    }
  }
}

// Per row: T (the k-th largest key), the keys == T still needed, and the
// ordered write.  The row's candidates come in units whose candidates lie
// packed in index order from the unit's first slot: below npacked, runs of
// `pack` chunks (the main scan kernel's rounds; pack = 1: every chunk of a
// compaction from scores), then single chunks (the scan's tail tiles).
//   counts — chunk counts and stamps read coalesced (thread c takes chunk c,
//            c + 1024, ...), summed per unit across the unit's lanes, then
//            prefixed over the units in index order;
//   load   — with at most kRegCand candidates the row's candidates, in index
//            order, are split into one contiguous segment per wave and loaded
//            64 at a time into registers (lane l of step j: candidate
//            s0 + 64 j + l of the wave's segment [s0, s1)), each candidate's
//            slot read from an LDS table the units' threads fill;
//   select — two radix digits counted from the cut into LDS give T and the
//            keys == T still needed; the keys > T and == T of every wave's
//            segment, prefixed over the waves, place every selected index
//            (every key > T, the earliest keys == T) at its position in index
//            order.
// A row whose cut failed (fewer than k candidates, a unit with more than its
// slots hold, a chunk stamped with another cut) is selected from the scores;
// a row with more candidates than the registers hold, from the candidate
// regions; both by the same workgroup with more passes.
// mode 0: every row; a row whose candidates cannot give the selection goes to
// the scores, or, when there are none (fathom_scan_topk without a score
// buffer), is flagged (kS_FAIL, and its group in gflag) for a second pass.
// mode 1: the flagged rows only, from the scores.
// flags: kResolveStamps — every chunk's stamp must equal the row's cut;
// kResolveOver — the row's overflow word is checked.
// pack is a power of two at most 64 and npacked a multiple of it, so a run's
// chunks c are consecutive lanes of one wave.
constexpr int kResolveStamps = 1, kResolveOver = 2;
constexpr int kRegSteps = 16;                              // loads of 64 candidates per wave
constexpr int kRegCand = kRegSteps * kResolveThreads;      // 16384 candidates at most
__global__ __launch_bounds__(kResolveThreads) void topk_resolve(const float* __restrict__ scores,
                                                                int64_t n, int64_t R, int k,
                                                                void* ws,
                                                                int32_t* __restrict__ out,
                                                                int mode, uint32_t* gflag,
                                                                int G, int pack, int64_t npacked,
                                                                int flags) {
  __shared__ uint32_t s_hist[2 * kBins];
  __shared__ uint32_t s_gt[kGroups];   // units' first candidates; groups' keys > T
  __shared__ uint32_t s_eq[kGroups];   // groups' keys == T
  __shared__ uint32_t s_addr[kRegCand];   // candidate f's slot in the candidate buffer
  __shared__ uint32_t s_tmp[kResolveThreads / 64];
  __shared__ uint32_t s_sel[2];
  const int64_t row = blockIdx.x;
  RowWs r = row_ws(ws, n, R, row);
  if (mode == 1 && r.st[kS_FAIL] == 0u) return;   // uniform over the workgroup
  ResolveSrc src;
  src.cand = reinterpret_cast<const uint2*>(r.cand);
  src.seg = r.seg;
  src.scores = scores + row * n;
  src.n = n;
  src.nc = n_chunks(n, R);
  src.R = R;
  src.region = r.region;
  const int64_t nc = src.nc;
  int32_t* dst = out + row * (int64_t)k;
  // The wave index, known to the compiler as uniform.
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = lane_id();
  constexpr int kW = kResolveThreads / 64;
  const uint64_t below = lanes_below();

  const int64_t nrun = npacked / pack;
  const int64_t nunits = nrun + (nc - npacked);
  const int lp = __builtin_ctz((unsigned)pack);
  const uint32_t cap = (uint32_t)pack * src.region;   // slots of a run
  auto unit_base = [&](int64_t u) {
    return u < nrun ? (uint32_t)u * cap : (uint32_t)(npacked + (u - nrun)) * src.region;
  };
  const uint32_t over = (flags & kResolveOver) ? r.st[kS_OVER] : 0u;
  const uint32_t tau = r.st[kS_TAU];

  // Counts.  Candidates per unit (s_gt[u] while they fit), the unit's limit
  // checked; then their prefix in s_gt and the total.
  const bool small = nunits <= kGroups;
  uint32_t ncand = 0;
  int stale = 0;
  {
    uint32_t mine = 0;
    // The loop bound is uniform: every lane takes part in the shuffles.
    for (int64_t c0 = 0; c0 < nc; c0 += 4 * kResolveThreads) {
      // Slices x of 1024 chunks that hold a chunk (uniform).
      const int nx = (int)min<int64_t>(4, (nc - c0 + kResolveThreads - 1) / kResolveThreads);
      uint32_t cnt[4] = {0u, 0u, 0u, 0u}, stp[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        if (x < nx) {
          const int64_t c = min<int64_t>(c0 + threadIdx.x + x * kResolveThreads, nc - 1);
          cnt[x] = r.seg[2 * c + 1];
          stp[x] = r.stamp[2 * c];
        }
      }
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int64_t c = c0 + threadIdx.x + x * kResolveThreads;
        const bool v = c < nc;
        const uint32_t t = v ? cnt[x] : 0u;
        if (v && (flags & kResolveStamps)) stale |= stp[x] != tau;
        uint32_t tr = t;   // the run's sum over its `pack` lanes
        for (int m = 1; m < pack; m <<= 1) tr += (uint32_t)__shfl_xor((int)tr, m);
        const bool packed = c < npacked;
        const int64_t u = packed ? (c >> lp) : nrun + (c - npacked);
        if (v && (!packed || (c & (pack - 1)) == 0)) {
          const uint32_t tot = packed ? tr : t;
          stale |= tot > (packed ? cap : src.region);   // more than the unit holds
          if (small) s_gt[u] = tot;
          mine += tot;
        }
      }
    }
    stale = __syncthreads_or(stale);
    uint32_t tot;
    if (small) {
      const int64_t per = (nunits + kResolveThreads - 1) / kResolveThreads;
      const int64_t u0 = min<int64_t>(nunits, threadIdx.x * per), u1 = min<int64_t>(nunits, u0 + per);
      uint32_t sum = 0;
      for (int64_t u = u0; u < u1; ++u) sum += s_gt[u];
      uint32_t run = block_exclusive_sum<kResolveThreads>(sum, s_tmp, tot);
      for (int64_t u = u0; u < u1; ++u) {
        const uint32_t t = s_gt[u];
        s_gt[u] = run;
        run += t;
      }
      __syncthreads();   // every unit's prefix is read by other threads below
    } else {
      (void)block_exclusive_sum<kResolveThreads>(mine, s_tmp, tot);
    }
    ncand = tot;
  }
  src.direct = ncand < (uint32_t)k || over != 0u || stale || mode == 1;   // the cut failed
  // Mode 0 records for every row whether the second pass must select it.
  // A row it need not select is recorded at the end: a barrier waits for
  // every global store in flight, so the store goes after the last one.
  const bool fail = src.direct && scores == nullptr;
  const bool record = mode == 0 && threadIdx.x == 0 && gflag != nullptr;
  if (fail) {   // no scores to fall back on: flag the row
    if (record) r.st[kS_FAIL] = 1u;
    if (threadIdx.x == 0) gflag[row / G] = 1u;
    return;
  }
  const bool regs = !src.direct && small && ncand <= (uint32_t)kRegCand;

  // T (the k-th largest of the keys visit(f) passes to f, once per digit) and
  // the keys == T to take.  from_tau: every key is >= tau and the cut sits
  // just below the k-th key, so bins of 4096 keys above tau (the last one
  // open-ended), then the 4096 keys of the chosen bin; otherwise, or when the
  // k-th key lies in the open-ended bin, three radix digits (11, 11, 10 bits)
  // from the top.
  auto kth = [&](auto&& visit, bool from_tau, uint32_t& T, uint32_t& need) {
    need = (uint32_t)k;
    uint32_t prefix = 0;
    bool done = false;
    if (from_tau) {
      for (int i = threadIdx.x; i < kBins; i += kResolveThreads) s_hist[i] = 0u;
      __syncthreads();
      visit([&](uint32_t key) { atomicAdd(&s_hist[min((key - tau) >> 12, (uint32_t)kBins - 1u)], 1u); });
      __syncthreads();
      {
        constexpr int kPer = kBins / kResolveThreads;
        uint32_t h[kPer];
#pragma unroll
        for (int b = 0; b < kPer; ++b) h[b] = s_hist[threadIdx.x * kPer + b];
        pick_bin<kResolveThreads, kPer>(h, need, s_tmp, s_sel);
      }
      __syncthreads();
      const uint32_t binA = s_sel[0], needA = s_sel[1];
      __syncthreads();
      if (binA < (uint32_t)kBins - 1u) {
        for (int i = threadIdx.x; i < 2 * kBins; i += kResolveThreads) s_hist[i] = 0u;
        __syncthreads();
        visit([&](uint32_t key) {
          const uint32_t d = key - tau;
          if ((d >> 12) == binA) atomicAdd(&s_hist[d & 4095u], 1u);
        });
        __syncthreads();
        constexpr int kPer = 2 * kBins / kResolveThreads;
        uint32_t h[kPer];
#pragma unroll
        for (int b = 0; b < kPer; ++b) h[b] = s_hist[threadIdx.x * kPer + b];
        pick_bin<kResolveThreads, kPer>(h, needA, s_tmp, s_sel);
        __syncthreads();
        prefix = tau + (binA << 12) + s_sel[0];
        need = s_sel[1];
        done = true;
        __syncthreads();
      }
    }
    for (int level = 0; level < 3 && !done; ++level) {
      const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
      const int bits = level == 2 ? 10 : 11;
      const int hi = shift + bits;   // bits at and above hi are fixed
      for (int i = threadIdx.x; i < kBins; i += kResolveThreads) s_hist[i] = 0u;
      __syncthreads();
      visit([&](uint32_t key) {
        const bool in = hi >= 32 || (key >> (hi & 31)) == (prefix >> (hi & 31));
        if (in) atomicAdd(&s_hist[(key >> shift) & ((1u << bits) - 1u)], 1u);
      });
      __syncthreads();
      constexpr int kPer = kBins / kResolveThreads;   // 2
      uint32_t h[kPer];
#pragma unroll
      for (int b = 0; b < kPer; ++b) {
        const int bin = threadIdx.x * kPer + b;
        h[b] = bin < (1 << bits) ? s_hist[bin] : 0u;
      }
      pick_bin<kResolveThreads, kPer>(h, need, s_tmp, s_sel);
      __syncthreads();
      prefix |= s_sel[0] << shift;
      need = s_sel[1];
      __syncthreads();
    }
    T = prefix;   // take every key > T and the first `need` keys == T
  };

  if (regs) {
    // Load.  s_addr[f]: the candidate buffer slot of candidate f (in index
    // order), written by the thread that owns f's unit, so that the loads'
    // addresses are one independent LDS read each.
    // Wave w fills its own run of consecutive units [w * upw, w * upw +
    // upw), 64 at a time: lane i reads the bounds of the i-th (consecutive
    // words: no LDS bank conflicts).  When none of the 64 holds more than 64
    // candidates (the fused call's rounds: about 17 each at q1m), lane i
    // writes its unit's entries itself, entry j of every unit in step j;
    // otherwise (fathom_topk's chunks: about 68 each) the wave writes each
    // unit's entries 64 at a time.
    const int64_t upw = (nunits + kW - 1) / kW;
    const int64_t wend = min<int64_t>(nunits, (int64_t)(wave + 1) * upw);
    for (int64_t ub = (int64_t)wave * upw; ub < wend; ub += 64) {
      const int64_t my = ub + lane;
      const bool ok = my < wend;
      const uint32_t ma = ok ? s_gt[my] : 0u;
      const uint32_t me = ok ? (my + 1 < nunits ? s_gt[my + 1] : ncand) : 0u;
      const uint32_t mb = ok ? unit_base(my) : 0u;
      const int nb = (int)min<int64_t>(64, wend - ub);   // >= 1
      // The bounds are in registers before the loop: without this wait the
      // loop would wait at every unit for the LDS writes of the one before.
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      const uint32_t cnt = me - ma;   // 0 past wend
      uint32_t mx = cnt;
      for (int o = 1; o < 64; o <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o));
      if (mx <= 64u) {   // uniform
        for (uint32_t j = 0; j < mx; ++j)
          if (j < cnt) s_addr[ma + j] = mb + j;
        continue;
      }
      // Four units at a time (the last one repeated past nb: the same
      // writes again); a unit's first 64 entries in one write, the rest of
      // a larger unit after.
      for (int i0 = 0; i0 < nb; i0 += 4) {
        uint32_t ua[4], ue[4], uw[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int i = min(i0 + x, nb - 1);
          ua[x] = (uint32_t)__builtin_amdgcn_readlane((int)ma, i);
          ue[x] = (uint32_t)__builtin_amdgcn_readlane((int)me, i);
          uw[x] = (uint32_t)__builtin_amdgcn_readlane((int)mb, i);
        }
#pragma unroll
        for (int x = 0; x < 4; ++x)
          if (ua[x] + (uint32_t)lane < ue[x]) s_addr[ua[x] + lane] = uw[x] + (uint32_t)lane;
#pragma unroll
        for (int x = 0; x < 4; ++x)
          for (uint32_t f = ua[x] + 64u + (uint32_t)lane; f < ue[x]; f += 64)
            s_addr[f] = uw[x] + (f - ua[x]);
      }
    }
    __syncthreads();
    const uint32_t seg = ((ncand + kW * 64 - 1) / (kW * 64)) * 64;
    const uint32_t s0 = min(ncand, (uint32_t)wave * seg), s1 = min(ncand, s0 + seg);
    const int steps = (int)((s1 - s0 + 63) / 64);   // uniform, at most kRegSteps
    uint2 e[kRegSteps];
    uint32_t vmask = 0;   // bit j: step j holds a candidate
    uint32_t addr[kRegSteps];
#pragma unroll
    for (int j = 0; j < kRegSteps; ++j) {   // every slot read first: one wait
      const uint32_t f = s0 + 64u * j + (uint32_t)lane;
      const bool v = f < s1;
      if (v) vmask |= 1u << j;
      addr[j] = s_addr[v ? f : 0u];
    }
#pragma unroll
    for (int j = 0; j < kRegSteps; ++j) {
      e[j] = make_uint2(0u, 0u);
      if (j < steps) e[j] = src.cand[addr[j]];   // uniform
    }
    uint32_t T, need;
    kth(
        [&](auto&& f) {
#pragma unroll
          for (int j = 0; j < kRegSteps; ++j)
            if (j < steps && ((vmask >> j) & 1u)) f(e[j].x);
        },
        true, T, need);
    // Keys > T and == T of each wave's segment (packed as gt | eq << 16, both
    // at most kRegCand < 2^16), prefixed over the waves; a key's output
    // position is (keys > T before it) + min(keys == T before it, need).
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kRegSteps; ++j) {
      if (j < steps) {   // uniform
        const bool v = (vmask >> j) & 1u;
        gt += (uint32_t)__popcll(__ballot(v && e[j].x > T));
        eq += (uint32_t)__popcll(__ballot(v && e[j].x == T));
      }
    }
    if (lane == 0) s_hist[wave] = gt | (eq << 16);
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += s_hist[w];
    uint32_t eq_seen = before >> 16;
    uint32_t pos = (before & 0xffffu) + min(eq_seen, need);
#pragma unroll
    for (int j = 0; j < kRegSteps; ++j) {
      if (j < steps) {   // uniform
        const bool v = (vmask >> j) & 1u;
        const bool g = v && e[j].x > T, q = v && e[j].x == T;
        const uint64_t eqm = __ballot(q);
        const bool take = g || (q && eq_seen + (uint32_t)__popcll(eqm & below) < need);
        const uint64_t tm = __ballot(take);
        const uint32_t p = pos + (uint32_t)__popcll(tm & below);
        if (take && p < (uint32_t)k) dst[p] = (int32_t)e[j].y;   // p < k by construction
        pos += (uint32_t)__popcll(tm);
        eq_seen += (uint32_t)__popcll(eqm);
      }
    }
    if (record) r.st[kS_FAIL] = 0u;
    return;
  }

  uint32_t T, need;
  kth([&](auto&& f) { for_each_key(src, [&](uint32_t key, uint32_t) { f(key); }); }, false, T,
      need);
  // The row's chunks in at most kGroups groups of consecutive chunks: the keys
  // > T and == T of every group, prefixed over the groups.
  const int64_t per_group = (nc + kGroups - 1) / kGroups;
  const int ngroups = (int)((nc + per_group - 1) / per_group);
  for (int g = threadIdx.x; g < ngroups; g += kResolveThreads) s_gt[g] = s_eq[g] = 0u;
  __syncthreads();
  for_each_key(src, [&](uint32_t key, uint32_t idx) {
    const int g = (int)((int64_t)(idx / R) / per_group);
    if (key > T) atomicAdd(&s_gt[g], 1u);
    if (key == T) atomicAdd(&s_eq[g], 1u);
  });
  __syncthreads();
  block_prefix_inplace<kResolveThreads>(s_gt, ngroups, s_tmp);
  block_prefix_inplace<kResolveThreads>(s_eq, ngroups, s_tmp);
  __syncthreads();
  // One wave per group writes its selected indices in index order.
  for (int g = wave; g < ngroups; g += kResolveThreads / 64) {
    uint32_t eq_seen = s_eq[g];
    uint32_t pos = s_gt[g] + min(eq_seen, need);
    walk_chunks(src, (int64_t)g * per_group, min<int64_t>(nc, (int64_t)(g + 1) * per_group),
                [&](uint32_t key, uint32_t idx, bool v) {
                  const bool gt = v && key > T, eq = v && key == T;
                  const uint64_t eqm = __ballot(eq);
                  const bool take = gt || (eq && eq_seen + (uint32_t)__popcll(eqm & below) < need);
                  const uint64_t tm = __ballot(take);
                  const uint32_t p = pos + (uint32_t)__popcll(tm & below);
                  if (take && p < (uint32_t)k) dst[p] = (int32_t)idx;   // p < k by construction
                  pos += (uint32_t)__popcll(tm);
                  eq_seen += (uint32_t)__popcll(eqm);
                });
  }
  if (record) r.st[kS_FAIL] = 0u;
}

hipError_t launch_resolve(const float* scores, int64_t rows, int64_t n, int64_t R, int k,
                          int32_t* indices, void* ws, int mode, uint32_t* gflag, int G, int pack,
                          int64_t npacked, int flags, hipStream_t stream) {
  if (pack < 1 || pack > 64 || (pack & (pack - 1)) != 0 || npacked % pack != 0)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_resolve, dim3((unsigned)rows), dim3(kResolveThreads), 0, stream, scores,
                     n, R, k, ws, indices, mode, gflag, G, pack, npacked, flags);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fused_resolve(const float* scores, int64_t rows, int64_t n, int64_t R, int k,
                                int32_t* indices, void* ws, int mode, uint32_t* gflag, int G,
                                int pack, int64_t npacked, hipStream_t stream) {
  return launch_resolve(scores, rows, n, R, k, indices, ws, mode, gflag, G, pack, npacked,
                        kResolveStamps | kResolveOver, stream);
}

size_t topk_workspace_bytes(int64_t rows, int64_t n, int k) {
  (void)k;
  const size_t bytes = (size_t)rows * row_words(n, kChunk) * sizeof(uint32_t);
  return (bytes + 255) & ~(size_t)255;
}

namespace {
std::atomic<uint32_t> g_topk_epoch{0};
std::atomic<int> g_topk_publish{1}, g_topk_spin{kTopkCutSpin};
}  // namespace

void set_topk_cut_hooks(int publish, int spin_limit) {
  g_topk_publish.store(publish);
  g_topk_spin.store(spin_limit);
}

hipError_t launch_topk(const float* scores, int64_t rows, int64_t n, int k, int32_t* indices,
                       void* ws, hipStream_t stream) {
  const int64_t R = kChunk, nc = n_chunks(n, R);
  const int64_t nwg = std::min<int64_t>(rows * nc, kMaxCompactWgs);
  const TopkCut cut{g_topk_epoch.fetch_add(1u) + 1u, g_topk_publish.load(), g_topk_spin.load()};
  hipLaunchKernelGGL(topk_cut_compact, dim3((unsigned)(rows + nwg)), dim3(kThreads), kCutHistBytes,
                     stream,
                     scores, rows, n, k, ws, nwg, cut);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_resolve(scores, rows, n, R, k, indices, ws, 0, nullptr, 1, 1, nc, kResolveStamps,
                        stream);
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on device `dev`, looked up on the first call
// for that device with it current (the caller's current device is restored).
hipError_t scratch_ptr(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_topk_noalloc(const float* scores, int64_t rows, int64_t n, int k,
                               int32_t* indices, hipStream_t stream) {
  if (topk_workspace_bytes(rows, n, k) > kNoAllocScratchBytes) return hipErrorInvalidValue;
  int dev = -1;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  void* ws = nullptr;
  if ((e = scratch_ptr(dev, &ws)) != hipSuccess) return e;
  // Every kernel of the selection writes what it later reads (the cut, and
  // every chunk's count and stamp), and the ready word carries the call's
  // epoch, so nothing of the previous call's contents needs clearing.
  return launch_topk(scores, rows, n, k, indices, ws, stream);
}

}  // namespace fathom
