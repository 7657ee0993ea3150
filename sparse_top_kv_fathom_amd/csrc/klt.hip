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
//   klt_cov   — per (chunk, group): the 128 x 128 sums of centred products,
//               one 8 x 8 tile per thread, tokens staged in LDS as fp64;
//   klt_eig   — per group, one 1024-thread workgroup: sums the chunks in a
//               fixed order, then cyclic Jacobi on the covariance (upper
//               triangle packed in LDS, fp64; the accumulated rotation in
//               LDS, fp32), 64 disjoint rotations per step in round-robin
//               order, sweeps until the off-diagonal mass falls below 1e-28
//               of the total; eigenvalues descending, each eigenvector
//               signed so that its first component of magnitude at least
//               1/(2 sqrt(d)) is positive.
// Rotation (fp32, order fixed):
//   k'_ij = fold over c ascending from +0 of fma(fl32(k_ic - mu_c), V_cj, .),
//   rounded to binary16 nearest-even;  q'_hj = the same fold of q_hc.
#include "fathom_internal.h"

namespace fathom {
namespace {

constexpr int kCovThreads = 256;
constexpr int kCovTok = 32;          // tokens staged per step of klt_cov
constexpr int kEigThreads = 1024;
constexpr int kPairs = kD / 2;       // disjoint rotations per Jacobi step
constexpr int kPacked = kD * (kD + 1) / 2;
constexpr int kMaxSweeps = 24;
constexpr int kRotThreads = 256;
constexpr int kRotTiles = 16;        // 64-token tiles per rotation workgroup
constexpr int kXPitch = kBlock + 4;  // floats per channel row of the staged tile

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
  double* mean;   // [groups][P][d]
  double* cov;    // [groups][P][d][d]
};

__host__ __device__ inline FitLayout fit_layout(void* ws, int64_t groups, int64_t P) {
  FitLayout L;
  L.mean = static_cast<double*>(ws);
  L.cov = L.mean + groups * P * kD;
  return L;
}

// Column sums of chunk blockIdx.x of group blockIdx.y.  Thread t sums
// channels 2(t % 64) and 2(t % 64) + 1 over every 4th token of the chunk.
__global__ __launch_bounds__(kCovThreads) void klt_mean(const uint16_t* __restrict__ k, int64_t n,
                                                        int64_t per, int64_t P, void* ws,
                                                        int64_t groups) {
  __shared__ double s_part[4][kD];
  const int64_t g = blockIdx.y, p = blockIdx.x;
  const int64_t t0 = p * per, t1 = min(n, t0 + per);
  const int cp = threadIdx.x & 63, r = threadIdx.x >> 6;
  double s0 = 0.0, s1 = 0.0;
  const uint32_t* rows = reinterpret_cast<const uint32_t*>(k + g * n * kD);
  for (int64_t t = t0 + r; t < t1; t += 4) {
    const uint32_t w = rows[t * (kD / 2) + cp];
    s0 += f16_to_f64((uint16_t)(w & 0xffffu));
    s1 += f16_to_f64((uint16_t)(w >> 16));
  }
  s_part[r][2 * cp] = s0;
  s_part[r][2 * cp + 1] = s1;
  __syncthreads();
  if (threadIdx.x < kD) {
    const int c = threadIdx.x;
    const double s = ((s_part[0][c] + s_part[1][c]) + s_part[2][c]) + s_part[3][c];
    fit_layout(ws, groups, P).mean[(g * P + p) * kD + c] = s;
  }
}

// Sums of centred products of chunk blockIdx.x of group blockIdx.y: thread t
// owns rows 8(t / 16) .. +7 and columns 8(t % 16) .. +7 of the 128 x 128 sum.
__global__ __launch_bounds__(kCovThreads) void klt_cov(const uint16_t* __restrict__ k, int64_t n,
                                                       int64_t per, int64_t P, void* ws,
                                                       int64_t groups) {
  __shared__ double s_mu[kD];
  __shared__ double s_x[kCovTok][kD];
  const int64_t g = blockIdx.y, p = blockIdx.x;
  const int64_t t0 = p * per, t1 = min(n, t0 + per);
  const FitLayout L = fit_layout(ws, groups, P);
  if (threadIdx.x < kD) {
    double s = 0.0;
    for (int64_t i = 0; i < P; ++i) s += L.mean[(g * P + i) * kD + threadIdx.x];
    s_mu[threadIdx.x] = s / (double)n;
  }
  const int ti = threadIdx.x >> 4, tj = threadIdx.x & 15;
  double acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.0;
  // Staging: thread t loads token t / 8 of the step, channels 16 (t % 8) .. +15.
  const int lt = threadIdx.x >> 3, lc = (threadIdx.x & 7) * 16;
  for (int64_t s0 = t0; s0 < t1; s0 += kCovTok) {
    __syncthreads();
    const int64_t tok = s0 + lt;
    if (tok < t1) {
      const uint4* src = reinterpret_cast<const uint4*>(k + (g * n + tok) * kD + lc);
      const uint4 w0 = src[0], w1 = src[1];
      const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s_x[lt][lc + 2 * e] = f16_to_f64((uint16_t)(w[e] & 0xffffu)) - s_mu[lc + 2 * e];
        s_x[lt][lc + 2 * e + 1] = f16_to_f64((uint16_t)(w[e] >> 16)) - s_mu[lc + 2 * e + 1];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) s_x[lt][lc + e] = 0.0;
    }
    __syncthreads();
    for (int u = 0; u < kCovTok; ++u) {
      double ra[8], cb[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) ra[a] = s_x[u][8 * ti + a];
#pragma unroll
      for (int b = 0; b < 8; ++b) cb[b] = s_x[u][8 * tj + b];
#pragma unroll
      for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = __builtin_fma(ra[a], cb[b], acc[a][b]);
    }
  }
  double* dst = L.cov + (g * P + p) * kD * kD;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) dst[(8 * ti + a) * kD + 8 * tj + b] = acc[a][b];
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
  const double inv = 1.0 / (double)(n - 1);
  for (int e = tid; e < kD * kD; e += kEigThreads) {
    const int r = e / kD, c = e % kD;
    if (r <= c) {
      double s = 0.0;
      for (int64_t i = 0; i < P; ++i) s += L.cov[(g * P + i) * kD * kD + e];
      s_a[tri(r, c)] = s * inv;
    }
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
      // A <- J^T A J, one 2 x 2 block (pair i, pair k), i <= k, per item.
      for (int e = tid; e < kPairs * kPairs; e += kEigThreads) {
        const int i = e / kPairs, kk = e % kPairs;
        if (i > kk) continue;
        const int p = s_p[i], q = s_q[i];
        if (i == kk) {
          const double apq = s_a[tri(p, q)], t = s_t[i];
          s_a[tri(p, p)] -= t * apq;
          s_a[tri(q, q)] += t * apq;
          s_a[tri(p, q)] = 0.0;
          continue;
        }
        const int p2 = s_p[kk], q2 = s_q[kk];
        const double ci = s_c[i], si = s_s[i], ck = s_c[kk], sk = s_s[kk];
        const int i00 = tri(p, p2), i01 = tri(p, q2), i10 = tri(q, p2), i11 = tri(q, q2);
        const double x00 = s_a[i00], x01 = s_a[i01], x10 = s_a[i10], x11 = s_a[i11];
        const double y00 = ci * x00 - si * x10, y01 = ci * x01 - si * x11;
        const double y10 = si * x00 + ci * x10, y11 = si * x01 + ci * x11;
        s_a[i00] = y00 * ck - y01 * sk;
        s_a[i01] = y00 * sk + y01 * ck;
        s_a[i10] = y10 * ck - y11 * sk;
        s_a[i11] = y10 * sk + y11 * ck;
      }
      // V <- V J: row r, pair i per item.
      for (int e = tid; e < kD * kPairs; e += kEigThreads) {
        const int r = e / kPairs, i = e % kPairs;
        const int p = s_p[i], q = s_q[i];
        const float c = (float)s_c[i], s = (float)s_s[i];
        const float vp = s_v[r][p], vq = s_v[r][q];
        s_v[r][p] = c * vp - s * vq;
        s_v[r][q] = s * vp + c * vq;
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

// Rotated keys of kRotTiles 64-token tiles of group blockIdx.y.  Thread t owns
// tokens 4 (t % 16) .. +3 and outputs 8 (t / 16) .. +7 of a tile.
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
  const int tq = tid & 15, jo = tid >> 4;
  const int lt = tid >> 2, lc = (tid & 3) * 32;       // staging: token, first channel
  const int64_t nb = n / kBlock;
  for (int64_t tile = (int64_t)blockIdx.x * kRotTiles;
       tile < min<int64_t>(nb, ((int64_t)blockIdx.x + 1) * kRotTiles); ++tile) {
    __syncthreads();
    const uint4* src = reinterpret_cast<const uint4*>(k + (g * n + tile * kBlock + lt) * kD + lc);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const uint4 w = src[v];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = lc + 8 * v + 2 * e;
        s_x[c][lt] = f16_to_f32((uint16_t)(ws[e] & 0xffffu)) - s_mu[c];
        s_x[c + 1][lt] = f16_to_f32((uint16_t)(ws[e] >> 16)) - s_mu[c + 1];
      }
    }
    __syncthreads();
    float acc[4][8];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 8; ++b) acc[a][b] = 0.0f;
    for (int c = 0; c < kD; ++c) {
      const float4 x = *reinterpret_cast<const float4*>(&s_x[c][4 * tq]);
      const float4 v0 = *reinterpret_cast<const float4*>(&s_v[c][8 * jo]);
      const float4 v1 = *reinterpret_cast<const float4*>(&s_v[c][8 * jo + 4]);
      const float xs[4] = {x.x, x.y, x.z, x.w};
      const float vs[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = __builtin_fmaf(xs[a], vs[b], acc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      uint32_t h[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        h[b] = (uint32_t)f32_to_f16_rne(acc[a][2 * b]) |
               ((uint32_t)f32_to_f16_rne(acc[a][2 * b + 1]) << 16);
      *reinterpret_cast<uint4*>(out + (g * n + tile * kBlock + 4 * tq + a) * kD + 8 * jo) =
          make_uint4(h[0], h[1], h[2], h[3]);
    }
  }
}

// Rotated queries: thread j of group blockIdx.x folds coordinate j of every head.
__global__ __launch_bounds__(kD) void klt_rotate_q(const float* __restrict__ q,
                                                   const float* __restrict__ basis, int G,
                                                   float* __restrict__ out) {
  const int64_t g = blockIdx.x;
  const int j = threadIdx.x;
  const float* V = basis + g * kD * kD;
  for (int h = 0; h < G; ++h) {
    const float* qh = q + (g * G + h) * kD;
    float acc = 0.0f;
    for (int c = 0; c < kD; ++c) acc = __builtin_fmaf(qh[c], V[c * kD + j], acc);
    out[(g * G + h) * kD + j] = acc;
  }
}

int64_t fit_chunks(int64_t groups, int64_t n) {
  const int64_t nb = n / kBlock;
  int64_t p = (512 + groups - 1) / groups;
  p = p < 32 ? p : 32;
  p = p < nb ? p : nb;
  return p > 1 ? p : 1;
}

}  // namespace

size_t klt_fit_workspace_bytes(int64_t groups, int64_t n) {
  const int64_t P = fit_chunks(groups, n);
  return (size_t)(groups * P * (kD + kD * kD)) * sizeof(double);
}

hipError_t launch_klt_fit(const uint16_t* k, int64_t groups, int64_t n, float* mu, float* basis,
                          float* lambda, void* ws, hipStream_t stream) {
  const int64_t P = fit_chunks(groups, n);
  const int64_t nb = n / kBlock;
  const int64_t per = (nb + P - 1) / P * kBlock;
  const dim3 grid((unsigned)P, (unsigned)groups);
  hipLaunchKernelGGL(klt_mean, grid, dim3(kCovThreads), 0, stream, k, n, per, P, ws, groups);
  hipLaunchKernelGGL(klt_cov, grid, dim3(kCovThreads), 0, stream, k, n, per, P, ws, groups);
  hipLaunchKernelGGL(klt_eig, dim3((unsigned)groups), dim3(kEigThreads), 0, stream, n, P,
                     (const void*)ws, groups, mu, basis, lambda);
  return hipGetLastError();
}

hipError_t launch_klt_rotate_keys(const uint16_t* k, const float* mu, const float* basis,
                                  int64_t groups, int64_t n, uint16_t* out, hipStream_t stream) {
  const int64_t nb = n / kBlock;
  const dim3 grid((unsigned)((nb + kRotTiles - 1) / kRotTiles), (unsigned)groups);
  hipLaunchKernelGGL(klt_rotate, grid, dim3(kRotThreads), 0, stream, k, mu, basis, n, out);
  return hipGetLastError();
}

hipError_t launch_klt_rotate_queries(const float* q, const float* basis, int64_t groups, int G,
                                     float* out, hipStream_t stream) {
  hipLaunchKernelGGL(klt_rotate_q, dim3((unsigned)groups), dim3(kD), 0, stream, q, basis, G, out);
  return hipGetLastError();
}

}  // namespace fathom
