// The KLT-rotated store on gfx950: the basis fit, the key rotation that feeds
// fathom_encode, and the query rotation that feeds fathom_plan / fathom_scan.
//
// "Fathom: Per-Query Read Depth for Sparse Decoding over Offloaded KV Caches",
// §3.5: for models without query/key normalisation the store holds the bit
// planes of the rotated keys (k - mu) V, V the eigenbasis of the keys'
// covariance, and the importance of rotated coordinate j is the water-filling
// rule's with the rotated queries q V and the eigenvalue lambda_j as the
// channel variance.  Nothing is truncated: all d rotated coordinates are
// stored.  Appendix D fits mu, V and lambda on the session's own keys.
//
// Fit (fp64):
//   klt_mean  — per (chunk of tokens, group): fp64 column sums;
//   klt_cov   — per (chunk, group): the upper triangle of the 128 x 128 sums
//               of centred products on the fp64 matrix cores: the 36
//               upper-triangle 16 x 16 tiles, 9 per wave, each a chain of
//               16 x 16 x 4 fp64 MFMAs over the chunk's tokens, which are
//               staged in LDS 64 at a time as centred fp64 values;
//   klt_reduce— per (element block, group): the partial sums added in a
//               fixed order, divided by n - 1;
//   klt_eig   — per group, one 1024-thread workgroup: cyclic Jacobi on the
//               covariance (upper triangle packed in LDS, fp64; the
//               accumulated rotation in LDS, fp32), 64 disjoint rotations
//               per step in round-robin order, sweeps until the off-diagonal
//               mass falls below 1e-28 of the total (at most 24); eigenvalues
//               descending, each eigenvector signed so that its first
//               component of magnitude at least 1/(2 sqrt(d)) is positive.
// Rotation (fp32, order fixed):
//   k'_ij = fold over c ascending from +0 of fma(fl32(k_ic - mu_c), V_cj, .),
//   rounded to binary16 nearest-even;  q'_hj = the same fold of q_hc.
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kCovThreads = 256;    // 4 waves, 9 of the 36 upper-triangle 16 x 16 tiles each
constexpr int kCovTiles = 36;
constexpr int kCovTok = 64;          // tokens staged per step of klt_cov
constexpr int kCovPitch = kD + 16;   // doubles per staged token row: the 4 rows a fragment
                                     // read spans start 32 banks apart
constexpr int kEigThreads = 1024;
constexpr int kPairs = kD / 2;       // disjoint rotations per Jacobi step
constexpr int kPacked = kD * (kD + 1) / 2;
constexpr int kMaxSweeps = 24;
constexpr int kRotThreads = 512;
constexpr int kRotTok = 128;         // tokens per rotation tile
constexpr int kRotTiles = 32;        // tiles per rotation workgroup
constexpr int kXPitch = kRotTok + 4; // floats per channel row of the staged tile

__device__ __forceinline__ double f16_to_f64(uint16_t h) {
  return (double)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ uint16_t f32_to_f16_rne(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// Packed upper triangle: element (a, b), a <= b.
__device__ __forceinline__ int tri(int a, int b) {
  return a <= b ? b * (b + 1) / 2 + a : a * (a + 1) / 2 + b;
}

struct FitLayout {
  double* mean;   // [groups][P][d]       column sums per chunk
  double* cov;    // [groups][P][d][d]    centred product sums per chunk (r <= c)
  double* csum;   // [groups][d][d]       the covariance (r <= c)
};

__host__ __device__ inline FitLayout fit_layout(void* ws, int64_t groups, int64_t P) {
  FitLayout L;
  L.mean = static_cast<double*>(ws);
  L.cov = L.mean + groups * P * kD;
  L.csum = L.cov + groups * P * kD * kD;
  return L;
}

// Column sums of chunk blockIdx.x of group blockIdx.y.  Thread t sums
// channels 8(t % 16) .. +7 over tokens t / 16, t / 16 + 16, ... of the chunk
// (16-byte loads, four rows in flight per thread).
__global__ __launch_bounds__(256) void klt_mean(const uint16_t* __restrict__ k, int64_t n,
                                                int64_t per, int64_t P, void* ws, int64_t groups) {
  __shared__ double s_part[16][kD];
  const int64_t g = blockIdx.y, p = blockIdx.x;
  const int64_t t0 = p * per, t1 = min(n, t0 + per);
  const int c8 = threadIdx.x & 15, r = threadIdx.x >> 4;
  double acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0;
  const uint4* rows = reinterpret_cast<const uint4*>(k + g * n * kD);
  int64_t t = t0 + r;
  for (; t + 48 < t1; t += 64) {
    uint4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) w[u] = rows[(t + 16 * u) * (kD / 8) + c8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t x[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += f16_to_f64((uint16_t)(x[e] & 0xffffu));
        acc[2 * e + 1] += f16_to_f64((uint16_t)(x[e] >> 16));
      }
    }
  }
  for (; t < t1; t += 16) {
    const uint4 w = rows[t * (kD / 8) + c8];
    const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += f16_to_f64((uint16_t)(x[e] & 0xffffu));
      acc[2 * e + 1] += f16_to_f64((uint16_t)(x[e] >> 16));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_part[r][8 * c8 + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < kD) {
    const int c = threadIdx.x;
    double s = 0.0;
    for (int i = 0; i < 16; ++i) s += s_part[i][c];
    fit_layout(ws, groups, P).mean[(g * P + p) * kD + c] = s;
  }
}

// Sums of centred products of chunk blockIdx.x of group blockIdx.y, on the
// fp64 matrix cores.  Tile (ti, tj), ti <= tj, of the 8 x 8 grid of 16 x 16
// tiles is C += X_i^T X_j over the chunk's tokens, four at a time:
// v_mfma_f64_16x16x4f64 takes A[r][k] and B[k][c] in lane 16 k + r (resp.
// 16 k + c) and leaves C[4 e + l / 16][l % 16] in element e of lane l.  With
// A = X_i^T and B = X_j both operands are the same fragment shape: lane
// 16 k + r holds X[token k][16 b + r] for channel block b, so a wave loads
// the 8 blocks' fragments of a step once and feeds its 9 tiles from them.
// Wave w takes tiles w, w + 4, ... of the 36 in row order.
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kCovTilesPerWave = kCovTiles / (kCovThreads / 64);

// Row and column block of upper-triangle tile idx, in row order.
constexpr int cov_tile_row(int idx) {
  int r = 0;
  while (idx >= 8 - r) {
    idx -= 8 - r;
    ++r;
  }
  return r;
}
constexpr int cov_tile_col(int idx) {
  int r = 0;
  while (idx >= 8 - r) {
    idx -= 8 - r;
    ++r;
  }
  return r + idx;
}
struct CovTileTable {
  int row[kCovTiles], col[kCovTiles];
  constexpr CovTileTable() : row(), col() {
    for (int i = 0; i < kCovTiles; ++i) {
      row[i] = cov_tile_row(i);
      col[i] = cov_tile_col(i);
    }
  }
};
constexpr CovTileTable kCovTable{};

// The staged tokens' MFMA steps for wave W's tiles W, W + 4, ... (their row
// and column blocks are compile-time constants, so the fragments are read
// straight from registers).
template <int W>
__device__ __forceinline__ void cov_steps(const double (*s_x)[kCovPitch], int lane,
                                          f64x4 (&acc)[kCovTilesPerWave]) {
#pragma unroll 2
  for (int k4 = 0; k4 < kCovTok; k4 += 4) {
    double f[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) f[b] = s_x[k4 + (lane >> 4)][16 * b + (lane & 15)];
#pragma unroll
    for (int u = 0; u < kCovTilesPerWave; ++u)
      acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(f[kCovTable.row[W + 4 * u]],
                                                    f[kCovTable.col[W + 4 * u]], acc[u], 0, 0, 0);
  }
}

template <int W>
__device__ __forceinline__ void cov_store(double* dst, int lane,
                                          const f64x4 (&acc)[kCovTilesPerWave]) {
#pragma unroll
  for (int u = 0; u < kCovTilesPerWave; ++u)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dst[(16 * kCovTable.row[W + 4 * u] + 4 * e + (lane >> 4)) * kD +
          16 * kCovTable.col[W + 4 * u] + (lane & 15)] = acc[u][e];
}

__global__ __launch_bounds__(kCovThreads) void klt_cov(const uint16_t* __restrict__ k, int64_t n,
                                                       int64_t per, int64_t P, void* ws,
                                                       int64_t groups) {
  __shared__ double s_mu[kD];
  __shared__ double s_x[kCovTok][kCovPitch];
  const int64_t g = blockIdx.y, p = blockIdx.x;
  const int64_t t0 = p * per, t1 = min(n, t0 + per);
  const FitLayout L = fit_layout(ws, groups, P);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (threadIdx.x < kD) {
    double s = 0.0;
    for (int64_t i = 0; i < P; ++i) s += L.mean[(g * P + i) * kD + threadIdx.x];
    s_mu[threadIdx.x] = s / (double)n;
  }
  f64x4 acc[kCovTilesPerWave];
#pragma unroll
  for (int u = 0; u < kCovTilesPerWave; ++u) acc[u] = f64x4{0.0, 0.0, 0.0, 0.0};
  // Staging: thread t converts token t / 4 of the step, channels
  // 32 (t % 4) .. +31 (four 16-byte loads), centred, to fp64.  The next
  // step's loads are issued before this step's products, so they are in
  // flight while the matrix cores work.
  const int lt = threadIdx.x >> 2, lc = (threadIdx.x & 3) * 32;
  auto load = [&](int64_t s0, uint4 (&v)[4]) {
    const int64_t tok = s0 + lt;
    if (tok < t1) {
      const uint4* src = reinterpret_cast<const uint4*>(k + (g * n + tok) * kD + lc);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = src[i];
    }
  };
  uint4 v[4];
  load(t0, v);
  for (int64_t s0 = t0; s0 < t1; s0 += kCovTok) {
    __syncthreads();   // the previous step's products are done with s_x
    if (s0 + lt < t1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = lc + 8 * i + 2 * e;
          s_x[lt][c] = f16_to_f64((uint16_t)(w[e] & 0xffffu)) - s_mu[c];
          s_x[lt][c + 1] = f16_to_f64((uint16_t)(w[e] >> 16)) - s_mu[c + 1];
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) s_x[lt][lc + e] = 0.0;
    }
    __syncthreads();
    if (s0 + kCovTok < t1) load(s0 + kCovTok, v);
    switch (wave) {
      case 0: cov_steps<0>(s_x, lane, acc); break;
      case 1: cov_steps<1>(s_x, lane, acc); break;
      case 2: cov_steps<2>(s_x, lane, acc); break;
      default: cov_steps<3>(s_x, lane, acc); break;
    }
  }
  double* dst = L.cov + (g * P + p) * kD * kD;
  switch (wave) {
    case 0: cov_store<0>(dst, lane, acc); break;
    case 1: cov_store<1>(dst, lane, acc); break;
    case 2: cov_store<2>(dst, lane, acc); break;
    default: cov_store<3>(dst, lane, acc); break;
  }
}

// The covariance: element e = blockIdx.x * 256 + t of group blockIdx.y (row
// e / 128, column e % 128, upper triangle only) summed over the P partials
// in index order, times 1 / (n - 1).
__global__ __launch_bounds__(256) void klt_reduce(int64_t n, int64_t P, void* ws, int64_t groups) {
  const int64_t g = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e / kD > e % kD) return;
  const FitLayout L = fit_layout(ws, groups, P);
  const double* src = L.cov + g * P * kD * kD + e;
  double s = 0.0;
  for (int64_t i = 0; i < P; ++i) s += src[i * kD * kD];
  L.csum[g * kD * kD + e] = s * (1.0 / (double)(n - 1));
}

// Sum over the workgroup in a fixed order (per-wave shuffles, then the waves
// in index order on thread 0); every thread gets the total.
__device__ double block_sum(double v, double* s_red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_down(v, o, 64);
  const int wave = threadIdx.x >> 6;
  if (lane_id() == 0) s_red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kEigThreads / 64; ++w) t += s_red[w];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kEigThreads) void klt_eig(int64_t n, int64_t P, const void* ws,
                                                       int64_t groups, float* __restrict__ mu,
                                                       float* __restrict__ basis,
                                                       float* __restrict__ lambda) {
  __shared__ double s_a[kPacked];
  __shared__ float s_v[kD][kD];
  __shared__ double s_c[kPairs], s_s[kPairs], s_t[kPairs];
  __shared__ int s_p[kPairs], s_q[kPairs];
  __shared__ double s_red[kEigThreads / 64];
  __shared__ double s_lam[kD];
  const int64_t g = blockIdx.x;
  const int tid = threadIdx.x;
  const FitLayout L = fit_layout(const_cast<void*>(ws), groups, P);

  if (tid < kD) {
    double s = 0.0;
    for (int64_t i = 0; i < P; ++i) s += L.mean[(g * P + i) * kD + tid];
    mu[g * kD + tid] = (float)(s / (double)n);
  }
  for (int e = tid; e < kD * kD; e += kEigThreads) {
    const int r = e / kD, c = e % kD;
    if (r <= c) s_a[tri(r, c)] = L.csum[g * kD * kD + e];
    s_v[r][c] = r == c ? 1.0f : 0.0f;
  }
  __syncthreads();

  for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
    double off = 0.0, tot = 0.0;
    for (int e = tid; e < kPacked; e += kEigThreads) {
      // e = b (b + 1) / 2 + a  with a <= b
      int b = (int)((__builtin_sqrt(8.0 * e + 1.0) - 1.0) * 0.5);
      while ((b + 1) * (b + 2) / 2 <= e) ++b;
      while (b * (b + 1) / 2 > e) --b;
      const int a = e - b * (b + 1) / 2;
      const double x = s_a[e];
      if (a != b) off += 2.0 * x * x;
      tot += a != b ? 2.0 * x * x : x * x;
    }
    off = block_sum(off, s_red);
    tot = block_sum(tot, s_red);
    if (!(off > 1e-28 * tot)) break;

    for (int step = 0; step < kD - 1; ++step) {
      if (tid < kPairs) {
        int p, q;
        if (tid == 0) {
          p = step;
          q = kD - 1;
        } else {
          p = (step + tid) % (kD - 1);
          q = (step - tid + (kD - 1)) % (kD - 1);
        }
        if (p > q) {
          const int x = p;
          p = q;
          q = x;
        }
        const double apq = s_a[tri(p, q)];
        double c = 1.0, s = 0.0, t = 0.0;
        if (apq != 0.0) {
          const double tau = (s_a[tri(q, q)] - s_a[tri(p, p)]) / (2.0 * apq);
          t = (tau >= 0.0 ? 1.0 : -1.0) / (__builtin_fabs(tau) + __builtin_sqrt(1.0 + tau * tau));
          c = 1.0 / __builtin_sqrt(1.0 + t * t);
          s = t * c;
        }
        s_p[tid] = p;
        s_q[tid] = q;
        s_c[tid] = c;
        s_s[tid] = s;
        s_t[tid] = t;
      }
      __syncthreads();
      // A <- J^T A J, one 2 x 2 block (pair i, pair k), i <= k, per item;
      // item e = tid + 1024 m has k = tid % 64 (fixed per thread) and
      // i = tid / 64 + 16 m.
      const int kk = tid & (kPairs - 1);
      const int p2 = s_p[kk], q2 = s_q[kk];
      const double ck = s_c[kk], sk = s_s[kk];
#pragma unroll
      for (int m = 0; m < kPairs * kPairs / kEigThreads; ++m) {
        const int i = (tid >> 6) + 16 * m;
        if (i > kk) continue;
        const int p = s_p[i], q = s_q[i];
        if (i == kk) {
          const double apq = s_a[tri(p, q)], t = s_t[i];
          s_a[tri(p, p)] -= t * apq;
          s_a[tri(q, q)] += t * apq;
          s_a[tri(p, q)] = 0.0;
          continue;
        }
        const double ci = s_c[i], si = s_s[i];
        const int i00 = tri(p, p2), i01 = tri(p, q2), i10 = tri(q, p2), i11 = tri(q, q2);
        const double x00 = s_a[i00], x01 = s_a[i01], x10 = s_a[i10], x11 = s_a[i11];
        const double y00 = ci * x00 - si * x10, y01 = ci * x01 - si * x11;
        const double y10 = si * x00 + ci * x10, y11 = si * x01 + ci * x11;
        s_a[i00] = y00 * ck - y01 * sk;
        s_a[i01] = y00 * sk + y01 * ck;
        s_a[i10] = y10 * ck - y11 * sk;
        s_a[i11] = y10 * sk + y11 * ck;
      }
      // V <- V J: item e = tid + 1024 m is row tid / 64 + 16 m of pair tid % 64.
      {
        const float c = (float)ck, sn = (float)sk;
#pragma unroll
        for (int m = 0; m < kD * kPairs / kEigThreads; ++m) {
          const int r = (tid >> 6) + 16 * m;
          const float vp = s_v[r][p2], vq = s_v[r][q2];
          s_v[r][p2] = c * vp - sn * vq;
          s_v[r][q2] = sn * vp + c * vq;
        }
      }
      __syncthreads();
    }
  }

  if (tid < kD) s_lam[tid] = s_a[tri(tid, tid)];
  __syncthreads();
  if (tid < kD) {
    const int j = tid;
    const double lj = s_lam[j];
    int rank = 0;
    for (int i = 0; i < kD; ++i) {
      const double li = s_lam[i];
      rank += (li > lj || (li == lj && i < j)) ? 1 : 0;
    }
    const float thr = 0.0441941738241592f;   // 1 / (2 sqrt(128))
    float sgn = 1.0f;
    for (int r = 0; r < kD; ++r) {
      const float v = s_v[r][j];
      if (__builtin_fabsf(v) >= thr) {
        sgn = v < 0.0f ? -1.0f : 1.0f;
        break;
      }
    }
    for (int r = 0; r < kD; ++r) basis[(g * kD + r) * kD + rank] = sgn * s_v[r][j];
    lambda[g * kD + rank] = (float)(lj > 0.0 ? lj : 0.0);
  }
}

// Rotated keys of kRotTiles 128-token tiles of group blockIdx.y.  Thread t
// (of 512: two waves per SIMD, the one workgroup its LDS lets a CU hold)
// owns tokens 8 (t % 16) .. +7 and outputs 4 (t / 16) .. +3 of a tile; per
// channel c it reads 8 centred values and 4 basis entries from LDS for 32
// fused multiply-adds.
__global__ __launch_bounds__(kRotThreads) void klt_rotate(const uint16_t* __restrict__ k,
                                                          const float* __restrict__ mu,
                                                          const float* __restrict__ basis,
                                                          int64_t n, uint16_t* __restrict__ out) {
  __shared__ float s_v[kD][kD];
  __shared__ float s_x[kD][kXPitch];
  __shared__ float s_mu[kD];
  const int64_t g = blockIdx.y;
  const int tid = threadIdx.x;
  const float4* vsrc = reinterpret_cast<const float4*>(basis + g * kD * kD);
  for (int e = tid; e < kD * kD / 4; e += kRotThreads)
    reinterpret_cast<float4*>(&s_v[0][0])[e] = vsrc[e];
  if (tid < kD) s_mu[tid] = mu[g * kD + tid];
  const int to = tid & 15, jo = tid >> 4;            // tokens 8 to .. +7, outputs 4 jo .. +3
  const int lt = tid >> 2, lc = (tid & 3) * 32;      // staging: token, first channel
  const int64_t ntile = (n + kRotTok - 1) / kRotTok;
  const int64_t t_begin = (int64_t)blockIdx.x * kRotTiles;
  const int64_t t_end = min<int64_t>(ntile, t_begin + kRotTiles);
  // The next tile's keys are loaded into registers while the current tile
  // is folded (the workgroup has the CU to itself: nothing else hides the
  // load); tokens past the row's end read the last token, and their
  // columns are folded and never written.
  uint4 pre[4];
  auto load_tile = [&](int64_t tile) {
    const int64_t tok = min<int64_t>(tile * kRotTok + lt, n - 1);
    const uint4* src = reinterpret_cast<const uint4*>(k + (g * n + tok) * kD + lc);
#pragma unroll
    for (int v = 0; v < 4; ++v) pre[v] = src[v];
  };
  if (t_begin < t_end) load_tile(t_begin);
  for (int64_t tile = t_begin; tile < t_end; ++tile) {
    const int64_t tok0 = tile * kRotTok;
    __syncthreads();   // the last tile's folds are done with s_x (s_mu is written)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint32_t ws[4] = {pre[v].x, pre[v].y, pre[v].z, pre[v].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = lc + 8 * v + 2 * e;
        s_x[c][lt] = f16_to_f32((uint16_t)(ws[e] & 0xffffu)) - s_mu[c];
        s_x[c + 1][lt] = f16_to_f32((uint16_t)(ws[e] >> 16)) - s_mu[c + 1];
      }
    }
    __syncthreads();
    if (tile + 1 < t_end) load_tile(tile + 1);
    float acc[8][4];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
#pragma unroll 4
    for (int c = 0; c < kD; ++c) {
      const float4 x0 = *reinterpret_cast<const float4*>(&s_x[c][8 * to]);
      const float4 x1 = *reinterpret_cast<const float4*>(&s_x[c][8 * to + 4]);
      const float4 v0 = *reinterpret_cast<const float4*>(&s_v[c][4 * jo]);
      const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      const float vs[4] = {v0.x, v0.y, v0.z, v0.w};
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_fmaf(xs[a], vs[b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      const int64_t tok = tok0 + 8 * to + a;
      if (tok >= n) break;
      const uint32_t h0 = (uint32_t)f32_to_f16_rne(acc[a][0]) |
                          ((uint32_t)f32_to_f16_rne(acc[a][1]) << 16);
      const uint32_t h1 = (uint32_t)f32_to_f16_rne(acc[a][2]) |
                          ((uint32_t)f32_to_f16_rne(acc[a][3]) << 16);
      *reinterpret_cast<uint2*>(out + (g * n + tok) * kD + 4 * jo) = make_uint2(h0, h1);
    }
  }
}

// Rotated queries of group blockIdx.x: the basis and the G query heads are
// staged in LDS with 16-byte loads, then thread t folds coordinate t % 128 of
// heads t / 128, t / 128 + 2, ...
__global__ __launch_bounds__(256) void klt_rotate_q(const float* __restrict__ q,
                                                    const float* __restrict__ basis, int G,
                                                    float* __restrict__ out) {
  __shared__ float s_v[kD][kD];
  __shared__ float s_q[8][kD];
  const int64_t g = blockIdx.x;
  const float4* vsrc = reinterpret_cast<const float4*>(basis + g * kD * kD);
  for (int e = threadIdx.x; e < kD * kD / 4; e += 256)
    reinterpret_cast<float4*>(&s_v[0][0])[e] = vsrc[e];
  for (int e = threadIdx.x; e < G * kD; e += 256) s_q[e / kD][e % kD] = q[g * G * kD + e];
  __syncthreads();
  const int j = threadIdx.x % kD;
  for (int h = threadIdx.x / kD; h < G; h += 2) {
    float acc = 0.0f;
    for (int c = 0; c < kD; ++c) acc = __builtin_fmaf(s_q[h][c], s_v[c][j], acc);
    out[(g * G + h) * kD + j] = acc;
  }
}

int64_t fit_chunks(int64_t groups, int64_t n) {
  const int64_t nb = n / kBlock;
  int64_t p = (512 + groups - 1) / groups;
  p = p < 64 ? p : 64;
  p = p < nb ? p : nb;
  return p > 1 ? p : 1;
}

}  // namespace

size_t klt_fit_workspace_bytes(int64_t groups, int64_t n) {
  const int64_t P = fit_chunks(groups, n);
  return (size_t)(groups * (P * kD + P * kD * kD + kD * kD)) * sizeof(double);
}

hipError_t launch_klt_fit(const uint16_t* k, int64_t groups, int64_t n, float* mu, float* basis,
                          float* lambda, void* ws, hipStream_t stream) {
  const int64_t P = fit_chunks(groups, n);
  const int64_t nb = n / kBlock;
  const int64_t per = (nb + P - 1) / P * kBlock;
  const dim3 grid((unsigned)P, (unsigned)groups);
  hipLaunchKernelGGL(klt_mean, grid, dim3(256), 0, stream, k, n, per, P, ws, groups);
  hipLaunchKernelGGL(klt_cov, grid, dim3(kCovThreads), 0, stream, k, n, per, P, ws, groups);
  hipLaunchKernelGGL(klt_reduce, dim3(kD * kD / 256, (unsigned)groups), dim3(256), 0, stream, n,
                     P, ws, groups);
  hipLaunchKernelGGL(klt_eig, dim3((unsigned)groups), dim3(kEigThreads), 0, stream, n, P,
                     (const void*)ws, groups, mu, basis, lambda);
  return hipGetLastError();
}

hipError_t launch_klt_rotate_keys(const uint16_t* k, const float* mu, const float* basis,
                                  int64_t groups, int64_t n, uint16_t* out, hipStream_t stream) {
  const int64_t ntile = (n + kRotTok - 1) / kRotTok;
  const dim3 grid((unsigned)((ntile + kRotTiles - 1) / kRotTiles), (unsigned)groups);
  hipLaunchKernelGGL(klt_rotate, grid, dim3(kRotThreads), 0, stream, k, mu, basis, n, out);
  return hipGetLastError();
}

hipError_t launch_klt_rotate_queries(const float* q, const float* basis, int64_t groups, int G,
                                     float* out, hipStream_t stream) {
  hipLaunchKernelGGL(klt_rotate_q, dim3((unsigned)groups), dim3(256), 0, stream, q, basis, G, out);
  return hipGetLastError();
}

}  // namespace fathom
