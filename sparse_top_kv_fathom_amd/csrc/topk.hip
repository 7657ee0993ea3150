// fathom_topk on gfx950: exact per-row top-k of fp32 scores.
//
// "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches",
// §2: the keys kept for attention are the top-k under the method's scores,
// chosen per query head.  Selection order: score descending, lower index
// first on equal scores; the k indices of a row are returned ascending.
//
// Radix select on an order-preserving 32-bit key (fp32 bits with the sign
// folded, -0 mapped to +0): three histogram passes over the row (11, 11 and
// 10 bits) each fix one digit of the k-th largest key T and how many keys
// equal to T are still needed.  A count pass records, per chunk of the row,
// how many keys are > T and == T; a per-row scan turns those into output
// offsets and per-chunk quotas of ties (the lowest indices win); a final
// pass writes every selected index at its rank, so the output comes out in
// index order with no sort.  Histograms are built in LDS per chunk and only
// non-empty bins are added to the row's global histogram.
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = 8192;             // keys per workgroup chunk
constexpr int kBins = 2048;              // widest digit (11 bits)
constexpr int kStateWords = 16;          // per-row state: [0] prefix, [1] need

struct RowWs {
  uint32_t* hist;    // [kBins]
  uint32_t* state;   // [kStateWords]
  uint32_t* cnt;     // [nchunks][2]: keys > T, keys == T
  uint32_t* off;     // [nchunks][2]: output base, quota of keys == T
};

__host__ __device__ inline int64_t n_chunks(int64_t n) { return (n + kChunk - 1) / kChunk; }

__host__ __device__ inline size_t row_ws_words(int64_t n) {
  return (size_t)kBins + kStateWords + (size_t)n_chunks(n) * 4;
}

__device__ inline RowWs row_ws(void* ws, int64_t n, int64_t row) {
  uint32_t* base = reinterpret_cast<uint32_t*>(ws) + row_ws_words(n) * row;
  RowWs r;
  r.hist = base;
  r.state = base + kBins;
  r.cnt = r.state + kStateWords;
  r.off = r.cnt + n_chunks(n) * 2;
  return r;
}

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) {
    const uint32_t o = __shfl_up(v, s, 64);
    if (lane >= s) v += o;
  }
  return v;
}

// Exclusive prefix sum over the workgroup; also returns the total.
__device__ __forceinline__ uint32_t block_exclusive_sum(uint32_t v, uint32_t* s_tmp,
                                                        uint32_t& total) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_sum(v);
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const uint32_t x = s_tmp[w];
    before += (w < wave) ? x : 0u;
    tot += x;
  }
  __syncthreads();
  total = tot;
  return before + inc - v;
}

__global__ __launch_bounds__(kThreads) void topk_init(void* ws, int64_t n, int k) {
  RowWs r = row_ws(ws, n, blockIdx.x);
  for (int i = threadIdx.x; i < kBins; i += kThreads) r.hist[i] = 0u;
  if (threadIdx.x == 0) {
    r.state[0] = 0u;
    r.state[1] = (uint32_t)k;
  }
}

// Histogram of digit (key >> SHIFT) & (2^BITS - 1) over the keys whose higher
// digits equal the prefix fixed so far.
template <int SHIFT, int BITS>
__global__ __launch_bounds__(kThreads) void topk_hist(const float* __restrict__ scores,
                                                      int64_t n, void* ws) {
  __shared__ uint32_t s_hist[1 << BITS];
  const int64_t row = blockIdx.y;
  RowWs r = row_ws(ws, n, row);
  for (int i = threadIdx.x; i < (1 << BITS); i += kThreads) s_hist[i] = 0u;
  const uint32_t prefix = r.state[0];
  __syncthreads();
  const float* src = scores + row * n;
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  const int64_t c1 = min<int64_t>(n, c0 + kChunk);
  constexpr int kHigh = SHIFT + BITS;
  for (int64_t i = c0 + threadIdx.x; i < c1; i += kThreads) {
    const uint32_t key = order_key(src[i]);
    const bool match = (kHigh >= 32) ? true : ((key >> (kHigh & 31)) == (prefix >> (kHigh & 31)));
    if (match) atomicAdd(&s_hist[(key >> SHIFT) & ((1u << BITS) - 1u)], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < (1 << BITS); i += kThreads) {
    const uint32_t c = s_hist[i];
    if (c != 0u) atomicAdd(&r.hist[i], c);
  }
}

// Pick the bin that holds the need-th largest remaining key; clear the
// histogram for the next digit.
template <int SHIFT, int BITS>
__global__ __launch_bounds__(kThreads) void topk_select(int64_t n, void* ws) {
  __shared__ uint32_t s_tmp[kThreads / 64];
  constexpr int kPer = (1 << BITS) / kThreads;
  RowWs r = row_ws(ws, n, blockIdx.x);
  const uint32_t need = r.state[1];
  uint32_t h[kPer];
  uint32_t mine = 0;
#pragma unroll
  for (int b = 0; b < kPer; ++b) {
    h[b] = r.hist[threadIdx.x * kPer + b];
    mine += h[b];
  }
  uint32_t total;
  const uint32_t before = block_exclusive_sum(mine, s_tmp, total);
  const uint32_t above = total - before - mine;  // keys in higher bins
  if (above < need && need <= above + mine) {
    uint32_t acc = above;
#pragma unroll
    for (int b = kPer - 1; b >= 0; --b) {
      if (acc + h[b] >= need) {
        r.state[0] |= (uint32_t)(threadIdx.x * kPer + b) << SHIFT;
        r.state[1] = need - acc;
        break;
      }
      acc += h[b];
    }
  }
#pragma unroll
  for (int b = 0; b < kPer; ++b) r.hist[threadIdx.x * kPer + b] = 0u;
}

// Per chunk: number of keys > T and == T.
__global__ __launch_bounds__(kThreads) void topk_count(const float* __restrict__ scores,
                                                       int64_t n, void* ws) {
  __shared__ uint32_t s_tmp[kThreads / 64];
  const int64_t row = blockIdx.y;
  RowWs r = row_ws(ws, n, row);
  const uint32_t T = r.state[0];
  const float* src = scores + row * n;
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  const int64_t c1 = min<int64_t>(n, c0 + kChunk);
  uint32_t gt = 0, eq = 0;
  for (int64_t i = c0 + threadIdx.x; i < c1; i += kThreads) {
    const uint32_t key = order_key(src[i]);
    gt += key > T;
    eq += key == T;
  }
  uint32_t tgt, teq;
  block_exclusive_sum(gt, s_tmp, tgt);
  block_exclusive_sum(eq, s_tmp, teq);
  if (threadIdx.x == 0) {
    r.cnt[blockIdx.x * 2 + 0] = tgt;
    r.cnt[blockIdx.x * 2 + 1] = teq;
  }
}

// Per row: output base of every chunk and its quota of keys equal to T (the
// earliest chunks take the ties first).
__global__ __launch_bounds__(kThreads) void topk_offsets(int64_t n, void* ws) {
  __shared__ uint32_t s_tmp[kThreads / 64];
  RowWs r = row_ws(ws, n, blockIdx.x);
  const uint32_t need = r.state[1];
  const int64_t nc = n_chunks(n);
  const int64_t per = (nc + kThreads - 1) / kThreads;
  const int64_t a = min<int64_t>(nc, threadIdx.x * per), b = min<int64_t>(nc, a + per);
  uint32_t gt = 0, eq = 0;
  for (int64_t c = a; c < b; ++c) {
    gt += r.cnt[c * 2 + 0];
    eq += r.cnt[c * 2 + 1];
  }
  uint32_t tot;
  uint32_t cum_gt = block_exclusive_sum(gt, s_tmp, tot);
  uint32_t cum_eq = block_exclusive_sum(eq, s_tmp, tot);
  for (int64_t c = a; c < b; ++c) {
    const uint32_t g = r.cnt[c * 2 + 0], e = r.cnt[c * 2 + 1];
    const uint32_t taken_before = min(cum_eq, need);
    const uint32_t quota = min(e, need - taken_before);
    r.off[c * 2 + 0] = cum_gt + taken_before;
    r.off[c * 2 + 1] = quota;
    cum_gt += g;
    cum_eq += e;
  }
}

// Ordered write: tiles of kThreads consecutive keys, one per thread.  A
// packed (gt, eq) prefix sum ranks the selected keys of the tile.
__global__ __launch_bounds__(kThreads) void topk_write(const float* __restrict__ scores,
                                                       int64_t n, int k, void* ws,
                                                       int32_t* __restrict__ out) {
  __shared__ uint32_t s_tmp[kThreads / 64];
  const int64_t row = blockIdx.y;
  RowWs r = row_ws(ws, n, row);
  const uint32_t T = r.state[0];
  uint32_t base = r.off[blockIdx.x * 2 + 0];
  uint32_t quota = r.off[blockIdx.x * 2 + 1];
  const float* src = scores + row * n;
  int32_t* dst = out + row * (int64_t)k;
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  const int64_t c1 = min<int64_t>(n, c0 + kChunk);
  for (int64_t t0 = c0; t0 < c1; t0 += kThreads) {
    const int64_t i = t0 + threadIdx.x;
    uint32_t key = 0u;
    if (i < c1) key = order_key(src[i]);
    const bool is_gt = (i < c1) && key > T;
    const bool is_eq = (i < c1) && key == T;
    const uint32_t packed = ((uint32_t)is_gt << 16) | (uint32_t)is_eq;
    uint32_t tot;
    const uint32_t pre = block_exclusive_sum(packed, s_tmp, tot);
    const uint32_t gt_before = pre >> 16, eq_before = pre & 0xffffu;
    const uint32_t eq_sel_before = min(eq_before, quota);
    const bool take = is_gt || (is_eq && eq_before < quota);
    const uint32_t pos = base + gt_before + eq_sel_before;
    if (take && pos < (uint32_t)k) dst[pos] = (int32_t)i;  // pos < k by construction
    const uint32_t tot_gt = tot >> 16, tot_eq = tot & 0xffffu;
    base += tot_gt + min(tot_eq, quota);
    quota -= min(tot_eq, quota);
  }
}

}  // namespace

size_t topk_workspace_bytes(int64_t rows, int64_t n, int k) {
  (void)k;
  const size_t bytes = (size_t)rows * row_ws_words(n) * sizeof(uint32_t);
  return (bytes + 255) & ~(size_t)255;
}

hipError_t launch_topk(const float* scores, int64_t rows, int64_t n, int k, int32_t* indices,
                       void* ws, hipStream_t stream) {
  const unsigned nc = (unsigned)n_chunks(n);
  const dim3 grid_rows((unsigned)rows), grid_chunks(nc, (unsigned)rows), blk(kThreads);
  hipLaunchKernelGGL(topk_init, grid_rows, blk, 0, stream, ws, n, k);
  hipLaunchKernelGGL((topk_hist<21, 11>), grid_chunks, blk, 0, stream, scores, n, ws);
  hipLaunchKernelGGL((topk_select<21, 11>), grid_rows, blk, 0, stream, n, ws);
  hipLaunchKernelGGL((topk_hist<10, 11>), grid_chunks, blk, 0, stream, scores, n, ws);
  hipLaunchKernelGGL((topk_select<10, 11>), grid_rows, blk, 0, stream, n, ws);
  hipLaunchKernelGGL((topk_hist<0, 10>), grid_chunks, blk, 0, stream, scores, n, ws);
  hipLaunchKernelGGL((topk_select<0, 10>), grid_rows, blk, 0, stream, n, ws);
  hipLaunchKernelGGL(topk_count, grid_chunks, blk, 0, stream, scores, n, ws);
  hipLaunchKernelGGL(topk_offsets, grid_rows, blk, 0, stream, n, ws);
  hipLaunchKernelGGL(topk_write, grid_chunks, blk, 0, stream, scores, n, k, ws, indices);
  return hipGetLastError();
}

}  // namespace fathom
