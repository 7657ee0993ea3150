// Per-row workspace of the top-k selection, shared by the top-k kernels and
// by the scan when it emits candidates itself.  Not part of the public ABI.
#pragma once

#include "fathom_internal.h"

namespace fathom {
namespace topk {

constexpr int kBins = 2048;           // radix digit: 11 bits
constexpr int kCompactChunk = 8192;   // keys per region when compacting from scores

// Per-row workspace (32-bit words).
enum : int {
  kS_TAU = 0,       // candidate cut
  kS_OVER,          // nonzero: a chunk had more candidates than its region
  kS_T,             // the k-th largest key (set by the resolve)
  kS_NEED,          // keys == T to take
  kS_FAIL,          // 1: fathom_scan_topk could not select from the candidates
  kS_READY,         // fathom_scan_topk: tau | 1 once the cut is published, else 0
  kS_WORDS = 16
};

// Candidates are kept per region of R consecutive keys of a row: R =
// kCompactChunk when compacting from scores, the scan's wave tile when the
// scan emits them.
__host__ __device__ inline int64_t n_chunks(int64_t n, int64_t R) { return (n + R - 1) / R; }

// Candidate buffer capacity of a row, shared equally by its chunks.
// Compaction from scores (R = kCompactChunk): n / 8, between 8192 and 65536
// keys (512 per 8192-key chunk at n = 2^20).  The scan's own candidates (R =
// its 512-key wave tile): n / 4, at least 8192 (128 per tile, 512 per
// 2048-key round), so that top keys crowded into one stretch of the row, up
// to a quarter of a round, still fit; only the candidates written cost time,
// not the capacity.
__host__ __device__ inline int64_t cand_cap(int64_t n, int64_t R) {
  if (R != kCompactChunk) return n / 4 < 8192 ? 8192 : n / 4;
  const int64_t c = n / 8;
  return c < 8192 ? 8192 : (c > 65536 ? 65536 : c);
}
__host__ __device__ inline uint32_t region(int64_t n, int64_t R) {
  return (uint32_t)(cand_cap(n, R) / n_chunks(n, R));
}

__host__ __device__ inline size_t row_words(int64_t n, int64_t R) {
  return kS_WORDS + 2 * (size_t)cand_cap(n, R) + 4 * (size_t)n_chunks(n, R);
}

struct RowWs {
  uint32_t* st;      // [kS_WORDS]
  uint32_t* cand;    // [nchunks][region][2]: key, index
  uint32_t* seg;     // [nchunks][2]: first slot of the chunk's candidates, their count
  uint32_t* stamp;   // [nchunks][2]: fathom_scan_topk: the cut chunk c was emitted with, at [2c]
  uint32_t region;
};

__device__ __forceinline__ RowWs row_ws(void* ws, int64_t n, int64_t R, int64_t row) {
  uint32_t* p = reinterpret_cast<uint32_t*>(ws) + row_words(n, R) * row;
  RowWs r;
  r.region = region(n, R);
  r.st = p;
  r.cand = r.st + kS_WORDS;
  r.seg = r.cand + 2 * (size_t)cand_cap(n, R);
  r.stamp = r.seg + 2 * (size_t)n_chunks(n, R);
  return r;
}

// The same layout from precomputed offsets (no division on the device): for
// kernels that address many rows.
struct RowGeom {
  uint64_t words;      // row_words(n, R)
  uint32_t region;     // region(n, R)
  uint32_t seg_off;    // first word of the segment table
  uint32_t stamp_off;  // first word of the stamp table
};
__host__ __device__ inline RowGeom row_geom(int64_t n, int64_t R) {
  RowGeom g;
  g.words = row_words(n, R);
  g.region = region(n, R);
  g.seg_off = (uint32_t)(kS_WORDS + 2 * cand_cap(n, R));
  g.stamp_off = g.seg_off + 2 * (uint32_t)n_chunks(n, R);
  return g;
}
__device__ __forceinline__ RowWs row_at(void* ws, const RowGeom& g, int64_t row) {
  uint32_t* p = reinterpret_cast<uint32_t*>(ws) + g.words * (uint64_t)row;
  RowWs r;
  r.region = g.region;
  r.st = p;
  r.cand = p + kS_WORDS;
  r.seg = p + g.seg_off;
  r.stamp = p + g.stamp_off;
  return r;
}

// Workspace of fathom_scan_topk: per-row selection state with one candidate
// region per scan wave tile (R = 512 keys), the sample's order keys, a flag
// per group (a row of the group must be selected again from its scores), and
// room for the scores of every row (used only when the caller passes no score
// buffer and a row's selection fails, or when the call cannot take the fused
// path).
constexpr int kMaxSampleKeys = 16384;   // sampled keys per row at most
constexpr int kSampleFlags = 64;        // sample workgroups per group at most
struct FusedWs {
  void* rows;        // [rows] RowWs with R = the scan's tile
  uint32_t* sample;  // [rows][kMaxSampleKeys] order keys of the sampled scores
  uint32_t* gflag;   // [groups]
  uint32_t* sflag;   // [groups][kSampleFlags] epoch of the call whose sample part is out
  float* scores;     // [rows][n]
};
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline size_t fused_front_bytes(int64_t rows, int64_t groups, int64_t n,
                                                    int64_t R) {
  // The fused layout, or fathom_topk's (used when the call is not fused),
  // whichever is larger; the score area follows.
  const size_t fused = align256((size_t)rows * row_words(n, R) * 4) +
                       align256((size_t)rows * kMaxSampleKeys * 4) +
                       align256((size_t)groups * (1 + kSampleFlags) * 4);
  const size_t plain = align256((size_t)rows * row_words(n, kCompactChunk) * 4);
  return fused > plain ? fused : plain;
}
__host__ __device__ inline FusedWs fused_ws(void* ws, int64_t rows, int64_t groups, int64_t n,
                                            int64_t R) {
  char* p = reinterpret_cast<char*>(ws);
  FusedWs f;
  f.rows = p;
  f.sample = reinterpret_cast<uint32_t*>(p + align256((size_t)rows * row_words(n, R) * 4));
  f.gflag = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(f.sample) +
                                        align256((size_t)rows * kMaxSampleKeys * 4));
  f.sflag = f.gflag + groups;
  f.scores = reinterpret_cast<float*>(p + fused_front_bytes(rows, groups, n, R));
  return f;
}

__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// The float whose order key is `key`; keys below that of -inf map to -inf
// and keys above that of +inf to a NaN, so `x >= key_float(key)` is
// `order_key(x) >= key` for every finite x.
__device__ __forceinline__ float key_float(uint32_t key) {
  if (key <= 0x007fffffu) return -__builtin_inff();
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

}  // namespace topk
}  // namespace fathom
