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
//   resolve — one workgroup per row: stages the candidates (key, index) in
//             LDS, finds the k-th largest key T with two radix digits counted
//             from tau and the keys == T still needed, counts per chunk the
//             keys > T and == T, prefixes the counts and writes every chunk's
//             selected indices (every key > T, the earliest keys == T) at its
//             prefix position, so the row comes out in index order without a
//             sort.
// If the cut fails (fewer than k keys >= tau, or a chunk with more than
// its region holds: heavy ties or adversarial rows), or the candidates do not
// fit in LDS, the resolve workgroup does all of it alone, from the scores or
// the regions: same result, many more passes.
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
constexpr int kLdsCand = 16320;                      // candidates staged in LDS at most

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

__device__ __forceinline__ int64_t key_index(int64_t c0, int i, int c) {
  const int wave = threadIdx.x >> 6, lane = lane_id();
  return c0 + (int64_t)wave * kWaveKeys + (int64_t)(i * 64 + lane) * 4 + c;
}

// FULL: the chunk lies inside the row and the row start is 16-byte aligned,
// so every key is valid and the loads are 16-byte vectors.
template <bool FULL>
__device__ __forceinline__ bool valid(int64_t c0, int i, int c, int64_t n) {
  return FULL || key_index(c0, i, c) < n;
}

__device__ __forceinline__ bool chunk_full(const float* src, int64_t n, int64_t c0) {
  return (reinterpret_cast<uintptr_t>(src) & 15) == 0 && c0 + kChunk <= n;
}

// Padding of a partial chunk reads -inf (never a candidate: see compact).
template <bool FULL>
__device__ __forceinline__ void load_vals(const float* __restrict__ src, int64_t n, int64_t c0,
                                          ChunkVals& V) {
  if (FULL) {
    typedef float f4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < kPerThread / 4; ++i) {
      const f4 x = __builtin_nontemporal_load(reinterpret_cast<const f4*>(src + key_index(c0, i, 0)));
      V.v[i][0] = x.x;
      V.v[i][1] = x.y;
      V.v[i][2] = x.z;
      V.v[i][3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPerThread / 4; ++i) {
      const int64_t e = key_index(c0, i, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) V.v[i][c] = (e + c < n) ? src[e + c] : -__builtin_inff();
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

// Per row: the cut tau from a sample of the row, in one workgroup: 16 runs of
// 1024 keys spread evenly over the row (the whole row when it has at most
// 16384 keys), held 16 per thread; tau = radix_cut of them at the target-th
// largest, target = the sample's share of k raised by 60% plus 16 keys (k
// itself for a whole row, where the cut then lies at or just below the k-th
// key).  Clears the row's overflow flag.
constexpr int kCutRuns = 16, kCutRun = 1024, kCutPer = kCutRuns * kCutRun / kResolveThreads;
static_assert(kCutPer == 16, "16 sampled keys per thread");

__global__ __launch_bounds__(kResolveThreads) void topk_cut(const float* __restrict__ scores,
                                                            int64_t n, int64_t R, int k,
                                                            void* ws) {
  __shared__ uint32_t s_hist[kBins];
  __shared__ uint32_t s_tmp[kResolveThreads / 64];
  __shared__ uint32_t s_sel[2];
  const int64_t row = blockIdx.x;
  RowWs r = row_ws(ws, n, R, row);
  const float* src = scores + row * n;
  const int tid = threadIdx.x;
  const bool whole = n <= (int64_t)kCutRuns * kCutRun;
  const int nkeys = whole ? (int)n : kCutRuns * kCutRun;
  uint32_t key[kCutPer];
  if (whole) {
#pragma unroll
    for (int u = 0; u < kCutPer; ++u) {
      const int64_t i = tid + (int64_t)u * kResolveThreads;
      key[u] = i < n ? order_key(src[i]) : 0u;
    }
  } else {
    // Run c = tid / 64 starts at c * (n - 1024) / 15 (rounded down to 4
    // keys); lane l takes its keys [16 l, 16 l + 16).
    const int64_t start = ((tid >> 6) * ((n - kCutRun) / (kCutRuns - 1))) & ~(int64_t)3;
    const float* p = src + start + (tid & 63) * kCutPer;
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
  const uint32_t prefix = radix_cut<kResolveThreads>(
      [&](auto&& f) {
#pragma unroll
        for (int u = 0; u < kCutPer; ++u)
          if (!whole || tid + (int64_t)u * kResolveThreads < n) f(key[u]);
      },
      need, s_hist, s_tmp, s_sel);
  if (tid == 0) {
    r.st[kS_TAU] = prefix;
    r.st[kS_OVER] = 0u;
  }
}

// Every key >= tau of one chunk written in index order to the chunk's region
// of the candidate buffer; the count goes to the segment table (a count above
// the region flags the row).  The test is a float compare against the cut
// (padding reads -inf: never >= a finite cut, and a cut of -inf's key only
// comes with whole-row sampling, where the cut is the low edge of a bin with
// keys); order keys are formed for candidates only.
template <bool F>
__device__ __forceinline__ void compact_chunk(const float* __restrict__ src, int64_t n, int64_t c0,
                                              const RowWs& r, uint32_t* s_cnt) {
  const float tauf = key_float(r.st[kS_TAU]);
  const int wave = threadIdx.x >> 6;
  ChunkVals V;
  load_vals<F>(src, n, c0, V);
  uint32_t ncand = 0;
#pragma unroll
  for (int i = 0; i < kPerThread / 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c)
      ncand += (uint32_t)__popcll(__ballot(V.v[i][c] >= tauf && valid<F>(c0, i, c, n)));
  if (lane_id() == 0) s_cnt[wave] = ncand;
  __syncthreads();
  const uint32_t base = (uint32_t)blockIdx.x * r.region;
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kWavesPerWg; ++w) t += s_cnt[w];
    r.seg[2 * blockIdx.x] = base;
    r.seg[2 * blockIdx.x + 1] = t;
    if (t > r.region) atomicOr(&r.st[kS_OVER], 1u);
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
        cand[c] = V.v[i][c] >= tauf && valid<F>(c0, i, c, n);
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
                make_uint2(order_key(V.v[i][c]), (uint32_t)key_index(c0, i, c));
          ++sl;
        }
      }
    }
  }
}

__global__ __launch_bounds__(kThreads) void topk_compact(const float* __restrict__ scores,
                                                         int64_t n, void* ws) {
  __shared__ uint32_t s_cnt[kWavesPerWg];
  const int64_t row = blockIdx.y;
  const RowWs r = row_ws(ws, n, kChunk, row);
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  const float* src = scores + row * n;
  if (chunk_full(src, n, c0)) compact_chunk<true>(src, n, c0, r, s_cnt);
  else compact_chunk<false>(src, n, c0, r, s_cnt);
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
// ordered write.  Rows whose candidates fit in LDS (the usual case) stage
// (key, index) there and do everything from LDS; other rows (the cut
// failed, or too many candidates or chunks) are resolved and written from the
// candidate regions or the scores, by the same workgroup.
// mode 0: every row; a row whose candidates cannot give the selection goes to
// the scores, or, when there are none (fathom_scan_topk without a score
// buffer), is flagged (kS_FAIL, and its group in gflag) for a second pass.
// mode 1: the flagged rows only, from the scores.
// pack > 1 (fathom_scan_topk): chunks [0, npacked) come in runs of `pack`
// whose candidates lie packed in index order from the run's first slot (the
// main scan kernel's rounds); the others each at their own first slot.
__global__ __launch_bounds__(kResolveThreads) void topk_resolve(const float* __restrict__ scores,
                                                                int64_t n, int64_t R, int k,
                                                                void* ws,
                                                                int32_t* __restrict__ out,
                                                                int mode, uint32_t* gflag,
                                                                int G, int pack, int64_t npacked) {
  __shared__ uint32_t s_hist[2 * kBins];
  __shared__ uint32_t s_gt[kGroups];
  // Staged candidates: keys and indices.  The path that does not stage them
  // uses s_idx as its per-group count of keys == T (kGroups <= kLdsCand).
  __shared__ uint32_t s_key[kLdsCand], s_idx[kLdsCand];
  static_assert(kGroups <= kLdsCand, "s_eq aliases s_idx");
  uint32_t* const s_eq = s_idx;
  // While staging: the first candidate slot of every chunk (s_hist is free).
  static_assert(kGroups <= 2 * kBins, "s_base aliases s_hist");
  uint32_t* const s_base = s_hist;
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
  const int wave = threadIdx.x >> 6, lane = lane_id();
  constexpr int kW = kResolveThreads / 64, kU = 8;

  // Candidates of the row: the chunk counts, summed (and, when they fit,
  // prefixed into s_gt for staging).  With at most 128 chunks, the first 128
  // candidate slots of the wave's chunks (w, w + 16, ...) are loaded at the
  // same time as the counts and the overflow flag, before either is known,
  // so staging them costs no second round trip to memory; slots past a
  // chunk's count are never used.  With packed runs (pack > 1) the same holds
  // for the first 32 slots of each run among the wave's first kPreRuns runs
  // (w, w + 16, ...: four runs of 16 lanes per load).
  const bool small = nc <= kGroups;
  const bool pre = pack == 1 && nc <= kW * kU;
  const bool ppre = pack > 1;
  constexpr int kPreRuns = 4 * kU;
  const int64_t nrun = npacked / pack;
  const uint32_t cap = (uint32_t)pack * src.region;   // slots of a run
  auto pre_run = [&](int i) { return wave + (int64_t)kW * (4 * i + (lane >> 4)); };
  uint32_t ncand = 0;
  const int64_t per = (nc + kResolveThreads - 1) / kResolveThreads;
  const int64_t c0 = min<int64_t>(nc, threadIdx.x * per), c1 = min<int64_t>(nc, c0 + per);
  const uint32_t first_count = c0 < c1 ? r.seg[2 * c0 + 1] : 0u;
  const uint32_t over = r.st[kS_OVER];
  // fathom_scan_topk (pack > 1): every tile stamps the cut it was emitted
  // with; a stamp other than the row's cut sends the row to the slow path.
  const uint32_t tau_row = r.st[kS_TAU];
  uint2 e[kU][2];
  if (pre) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t c = wave + u * kW;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t o = lane + 64 * h;
        e[u][h] = (c < nc && o < src.region) ? src.cand[(uint32_t)c * src.region + o]
                                             : make_uint2(0u, 0u);
      }
    }
  } else if (ppre) {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int64_t run = pre_run(i);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t o = (lane & 15) + 16 * h;
        e[i][h] = (run < nrun && o < cap) ? src.cand[(uint32_t)run * cap + o] : make_uint2(0u, 0u);
      }
    }
  }
  // Chunks past the packed runs (the scan's tail tiles, each at its own
  // slots chunk * region): wave w < their number prefetches the first 64 of
  // chunk npacked + w.
  const int64_t ntail = nc - npacked;
  const bool tpre = ppre && ntail <= kW;
  uint2 et = make_uint2(0u, 0u);
  if (tpre && wave < ntail && (uint32_t)lane < src.region)
    et = src.cand[(uint32_t)(npacked + wave) * src.region + lane];
  int stale = 0;
  {
    uint32_t mine = 0;
    for (int64_t c = c0; c < c1; ++c) {
      const uint32_t t = c == c0 ? first_count : r.seg[2 * c + 1];
      if (pack > 1) stale |= r.stamp[2 * c] != tau_row;
      if (small) {
        s_gt[c] = t;
        s_base[c] = r.seg[2 * c];
      }
      mine += t;
    }
    stale = __syncthreads_or(stale);
    uint32_t tot;
    uint32_t run = block_exclusive_sum<kResolveThreads>(mine, s_tmp, tot);
    ncand = tot;
    if (small)
      for (int64_t c = c0; c < c1; ++c) {
        const uint32_t t = s_gt[c];
        s_gt[c] = run;   // first LDS slot of chunk c
        run += t;
      }
  }
  src.direct = ncand < (uint32_t)k || over != 0u || stale || mode == 1;   // the cut failed
  // Mode 0 records for every row whether the second pass must select it.
  const bool fail = src.direct && scores == nullptr;
  if (mode == 0 && threadIdx.x == 0 && gflag != nullptr) r.st[kS_FAIL] = fail ? 1u : 0u;
  if (fail) {   // no scores to fall back on: flag the row
    if (threadIdx.x == 0) gflag[row / G] = 1u;
    return;
  }
  const bool lds = !src.direct && small && ncand <= (uint32_t)kLdsCand;
  __syncthreads();

  // Candidates of packed run `run`: first LDS slot and count.
  auto run_span = [&](int64_t run, uint32_t& d) {
    const int64_t ca = run * pack, cb = ca + pack;
    d = s_gt[ca];
    return (cb < nc ? s_gt[cb] : ncand) - d;
  };
  if (lds && ppre) {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int64_t run = pre_run(i);
      if (run < nrun) {
        uint32_t d;
        const uint32_t cnt = run_span(run, d);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t o = (lane & 15) + 16 * h;
          if (o < cnt) {
            s_key[d + o] = e[i][h].x;
            s_idx[d + o] = e[i][h].y;
          }
        }
      }
    }
  }
  if (lds && tpre && wave < ntail) {
    const int64_t c = npacked + wave;
    const uint32_t d = s_gt[c], cnt = (c + 1 < nc ? s_gt[c + 1] : ncand) - d;
    if ((uint32_t)lane < cnt) {
      s_key[d + lane] = et.x;
      s_idx[d + lane] = et.y;
    }
    for (uint32_t o = 64 + lane; o < cnt; o += 64) {
      const uint2 x = src.cand[(uint32_t)c * src.region + o];
      s_key[d + o] = x.x;
      s_idx[d + o] = x.y;
    }
  }
  if (lds && pre) {
    auto count = [&](int64_t c) { return (c + 1 < nc ? s_gt[c + 1] : ncand) - s_gt[c]; };
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t c = wave + u * kW;
      const uint32_t cnt = c < nc ? count(c) : 0u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t o = lane + 64 * h;
        if (o < cnt) {
          s_key[s_gt[c] + o] = e[u][h].x;
          s_idx[s_gt[c] + o] = e[u][h].y;
        }
      }
    }
  }
  if (lds) {
    // Stage the candidates, chunk after chunk in index order: chunk c at
    // [s_gt[c], s_gt[c] + count(c)).  With at most 128 chunks the first 128
    // candidates of every chunk were loaded above; any rest follows, wave w
    // taking chunks w, w + 16, ...  Otherwise the staging goes by units of
    // chunks whose candidates are contiguous (below).
    auto count = [&](int64_t c) { return (c + 1 < nc ? s_gt[c + 1] : ncand) - s_gt[c]; };
    if (pre) {
      for (int64_t c = wave; c < nc; c += kW)
        for (uint32_t o = 128 + lane; o < count(c); o += 64) {
          const uint2 e = src.cand[(uint32_t)c * src.region + o];
          s_key[s_gt[c] + o] = e.x;
          s_idx[s_gt[c] + o] = e.y;
        }
    } else {
      // Runs prefetched above: the candidates past their first 32.
      const int64_t ufirst = ppre ? min<int64_t>(nrun, (int64_t)kW * kPreRuns) : 0;
      if (ppre) {
        // Lane j < kPreRuns checks run w + 16 j; only runs with more than 32
        // candidates (rare) are visited.
        static_assert(kPreRuns <= 64, "one lane per prefetched run");
        const int64_t myrun = wave + (int64_t)kW * lane;
        uint32_t myd = 0, mycnt = 0;
        if (lane < kPreRuns && myrun < nrun) mycnt = run_span(myrun, myd);
        uint64_t big = __ballot(mycnt > 32u);
        while (big != 0ull) {
          const int j = __builtin_ctzll(big);
          big &= big - 1;
          const int64_t run = wave + (int64_t)kW * j;
          const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)myd, j);
          const uint32_t cnt = (uint32_t)__builtin_amdgcn_readlane((int)mycnt, j);
          for (uint32_t o = 32 + lane; o < cnt; o += 64) {
            const uint2 e = src.cand[(uint32_t)run * cap + o];
            s_key[d + o] = e.x;
            s_idx[d + o] = e.y;
          }
        }
      }
      // The other staging units: below npacked a run of `pack` chunks (its
      // candidates packed from the run's first slot, in index order), above it
      // single chunks.  Wave w copies units ufirst + w, ufirst + w + 16, ...,
      // kUU of them at a time, each in one piece of up to 128 candidates (the
      // rest of a larger unit follows).
      const int64_t nunits = tpre ? nrun : nrun + (nc - npacked);   // tail chunks done above
      constexpr int kUU = 8;
      for (int64_t u0 = ufirst + wave; u0 < nunits; u0 += kW * kUU) {
        uint32_t d[kUU], cnt[kUU], b[kUU];
        uint2 ev[kUU][2];
#pragma unroll
        for (int x = 0; x < kUU; ++x) {
          const int64_t u = u0 + x * kW;
          const int64_t ca = u < nrun ? u * pack : npacked + (u - nrun);
          const int64_t cb = u < nrun ? ca + pack : ca + 1;
          const bool v = u < nunits;
          d[x] = v ? s_gt[ca] : 0u;
          cnt[x] = v ? (cb < nc ? s_gt[cb] : ncand) - d[x] : 0u;
          b[x] = v ? s_base[ca] : 0u;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t o = lane + 64 * h;
            ev[x][h] = o < cnt[x] ? src.cand[b[x] + o] : make_uint2(0u, 0u);
          }
        }
#pragma unroll
        for (int x = 0; x < kUU; ++x) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t o = lane + 64 * h;
            if (o < cnt[x]) {
              s_key[d[x] + o] = ev[x][h].x;
              s_idx[d[x] + o] = ev[x][h].y;
            }
          }
          for (uint32_t o = 128 + lane; o < cnt[x]; o += 64) {
            const uint2 e = src.cand[b[x] + o];
            s_key[d[x] + o] = e.x;
            s_idx[d[x] + o] = e.y;
          }
        }
      }
    }
  }
  __syncthreads();

  uint32_t need = (uint32_t)k;
  uint32_t prefix = 0;
  bool done = false;
  if (lds) {
    // Candidates are keys >= tau and the cut sits just below the k-th key:
    // bins of 4096 keys above tau (the last one open-ended), then the 4096
    // keys of the chosen bin.
    const uint32_t tau = r.st[kS_TAU];
    for (int i = threadIdx.x; i < kBins; i += kResolveThreads) s_hist[i] = 0u;
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < ncand; i += kResolveThreads)
      atomicAdd(&s_hist[min((s_key[i] - tau) >> 12, (uint32_t)kBins - 1u)], 1u);
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
      for (uint32_t i = threadIdx.x; i < ncand; i += kResolveThreads) {
        const uint32_t d = s_key[i] - tau;
        if ((d >> 12) == binA) atomicAdd(&s_hist[d & 4095u], 1u);
      }
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
  // f(key, index) over every key the row selects among (LDS: the index is
  // not needed, 0 is passed).
  auto keys = [&](auto&& f) {
    if (lds) {
      for (uint32_t i = threadIdx.x; i < ncand; i += kResolveThreads) f(s_key[i], 0u);
    } else {
      for_each_key(src, f);
    }
  };
  // Three radix digits (11, 11, 10 bits), from the top.
  for (int level = 0; level < 3 && !done; ++level) {
    const int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    const int bits = level == 2 ? 10 : 11;
    const int hi = shift + bits;   // bits at and above hi are fixed
    for (int i = threadIdx.x; i < kBins; i += kResolveThreads) s_hist[i] = 0u;
    __syncthreads();
    keys([&](uint32_t key, uint32_t) {
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
  const uint32_t T = prefix;   // take every key > T and the first `need` keys == T

  // The row's chunks in at most kGroups groups of consecutive chunks: the keys
  // > T and == T of every group, prefixed over the groups.
  const int64_t per_group = (nc + kGroups - 1) / kGroups;
  const int ngroups = (int)((nc + per_group - 1) / per_group);
  if (lds) {
    // The staged candidates are in index order, so the selection is written
    // from one flat pass: wave w takes a contiguous segment of them, 64 at a
    // time; its counts of keys > T and == T (packed as gt | eq << 16, both
    // at most kLdsCand < 2^16) are prefixed over the waves, and a key's
    // output position is (keys > T before it) + min(keys == T before it,
    // need).
    const uint32_t seg = ((ncand + kW * 64 - 1) / (kW * 64)) * 64;
    const uint32_t s0 = min(ncand, (uint32_t)wave * seg), s1 = min(ncand, s0 + seg);
    uint32_t gt = 0, eq = 0;
    for (uint32_t o = s0; o < s1; o += 64) {
      const bool v = o + lane < s1;
      const uint32_t key = v ? s_key[o + lane] : 0u;
      gt += (uint32_t)__popcll(__ballot(v && key > T));
      eq += (uint32_t)__popcll(__ballot(v && key == T));
    }
    if (lane == 0) s_hist[wave] = gt | (eq << 16);
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += s_hist[w];
    const uint64_t below = lanes_below();
    uint32_t eq_seen = before >> 16;
    uint32_t pos = (before & 0xffffu) + min(eq_seen, need);
    for (uint32_t o = s0; o < s1; o += 64) {
      const bool v = o + lane < s1;
      const uint2 e = v ? make_uint2(s_key[o + lane], s_idx[o + lane]) : make_uint2(0u, 0u);
      const bool g = v && e.x > T, q = v && e.x == T;
      const uint64_t eqm = __ballot(q);
      const bool take = g || (q && eq_seen + (uint32_t)__popcll(eqm & below) < need);
      const uint64_t tm = __ballot(take);
      const uint32_t p = pos + (uint32_t)__popcll(tm & below);
      if (take && p < (uint32_t)k) dst[p] = (int32_t)e.y;   // p < k by construction
      pos += (uint32_t)__popcll(tm);
      eq_seen += (uint32_t)__popcll(eqm);
    }
    return;
  } else {
    for (int g = threadIdx.x; g < ngroups; g += kResolveThreads) s_gt[g] = s_eq[g] = 0u;
    __syncthreads();
    for_each_key(src, [&](uint32_t key, uint32_t idx) {
      const int g = (int)((int64_t)(idx / R) / per_group);
      if (key > T) atomicAdd(&s_gt[g], 1u);
      if (key == T) atomicAdd(&s_eq[g], 1u);
    });
  }
  __syncthreads();
  block_prefix_inplace<kResolveThreads>(s_gt, ngroups, s_tmp);
  block_prefix_inplace<kResolveThreads>(s_eq, ngroups, s_tmp);
  __syncthreads();
  const uint64_t below = lanes_below();
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
}

}  // namespace

hipError_t launch_fused_resolve(const float* scores, int64_t rows, int64_t n, int64_t R, int k,
                                int32_t* indices, void* ws, int mode, uint32_t* gflag, int G,
                                int pack, int64_t npacked, hipStream_t stream) {
  hipLaunchKernelGGL(topk_resolve, dim3((unsigned)rows), dim3(kResolveThreads), 0, stream, scores,
                     n, R, k, ws, indices, mode, gflag, G, pack, npacked);
  return hipGetLastError();
}

size_t topk_workspace_bytes(int64_t rows, int64_t n, int k) {
  (void)k;
  const size_t bytes = (size_t)rows * row_words(n, kChunk) * sizeof(uint32_t);
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_topk(const float* scores, int64_t rows, int64_t n, int k, int32_t* indices,
                       void* ws, hipStream_t stream) {
  const int64_t R = kChunk, nc = n_chunks(n, R);
  const dim3 grid_rows((unsigned)rows), grid_chunks((unsigned)nc, (unsigned)rows);
  hipLaunchKernelGGL(topk_cut, grid_rows, dim3(kResolveThreads), 0, stream, scores, n, R, k, ws);
  hipLaunchKernelGGL(topk_compact, grid_chunks, dim3(kThreads), 0, stream, scores, n, ws);
  hipLaunchKernelGGL(topk_resolve, grid_rows, dim3(kResolveThreads), 0, stream, scores, n, R, k,
                     ws, indices, 0, (uint32_t*)nullptr, 1, 1, (int64_t)0);
  return hipGetLastError();
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
  // Every kernel of the selection writes what it later reads (the cut and
  // the overflow flag set by the cut kernel, every chunk's count by the
  // compaction), so nothing of the previous call's contents needs clearing.
  return launch_topk(scores, rows, n, k, indices, ws, stream);
}

}  // namespace fathom
