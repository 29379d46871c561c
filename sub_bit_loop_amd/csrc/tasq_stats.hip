// Statistics for the pre-transform's channel permutation: mean and
// covariance, in fp64, of the scaled keys y = w * k / sigma (the transform
// before its permutation) with the T_c steps of a block stacked into one
// T_c*D vector, per (kv-head, block), over every (batch entry, token).
//
// LoopVQ review (arXiv 2611.05304), section 3.3: the permutation is taken from
// the T_c*D x T_c*D covariance of a block's stacked step keys.  Feature index
// s*D + d is channel d at block step s.  The bf16 keys, the fp32 weights and
// the fp16 sigma are exact in fp64; y is (w * k) / sigma rounded once.
#include "common.h"
#include "kernels.h"

namespace loopvq {

namespace {

__device__ __forceinline__ double scaled_key(const TasqStatsArgs& a, int h, int beta, int b, int j, int f) {
  const int s = f / a.D, d = f - s * a.D;
  const int t = beta * a.T_c + s;
  const uint16_t* row = a.x + b * a.xs0 + h * a.xs1 + t * a.xs2 + (int64_t)j * a.xs3;
  const double k = (double)bf16_to_f32(row[d]);
  const double sg = f16_bits_to_f64(a.sigma[((int64_t)b * a.sig_cap + j) * a.T + t]);
  return ((double)a.w[h * a.D + d] * k) / sg;
}

}  // namespace

// One workgroup per (kv-head, block), one thread per feature; tokens in
// (batch entry, token) order.
__global__ __launch_bounds__(1024) void tasq_mean_kernel(TasqStatsArgs a) {
  const int hb = blockIdx.x, h = hb / a.n_blk, beta = hb - h * a.n_blk;
  const int F = a.T_c * a.D;
  const int f = threadIdx.x;
  if (f >= F) return;
  double sum = 0.0;
  for (int b = 0; b < a.B; ++b)
    for (int j = 0; j < a.N; ++j) sum += scaled_key(a, h, beta, b, j, f);
  a.mean[(int64_t)hb * F + f] = sum / ((double)a.B * (double)a.N);
}

// 64 x 64 tile of the covariance per workgroup (256 threads, 4 x 4 entries
// each); tokens are staged 32 at a time in LDS as centred fp64 values.
constexpr int kCovTile = 64, kCovTok = 32;

__global__ __launch_bounds__(256) void tasq_cov_kernel(TasqStatsArgs a) {
  __shared__ double s_i[kCovTok][kCovTile];
  __shared__ double s_j[kCovTok][kCovTile];
  const int F = a.T_c * a.D;
  const int nt = F / kCovTile;
  const int ti = blockIdx.x / nt, tj = blockIdx.x - ti * nt;
  const int hb = blockIdx.y, h = hb / a.n_blk, beta = hb - h * a.n_blk;
  const double* mu = a.mean + (int64_t)hb * F;
  const int tid = threadIdx.x;
  const int ri = (tid >> 4) * 4, rj = (tid & 15) * 4;   // this thread's 4 x 4 block of the tile
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
  const int64_t n = (int64_t)a.B * a.N;
  for (int64_t t0 = 0; t0 < n; t0 += kCovTok) {
    // stage: 32 tokens x 64 features of both ranges (8 values per thread each)
    for (int e = tid; e < kCovTok * kCovTile; e += 256) {
      const int tk = e / kCovTile, fo = e - tk * kCovTile;
      const int64_t tt = t0 + tk;
      double yi = 0.0, yj = 0.0;
      if (tt < n) {
        const int b = (int)(tt / a.N), j = (int)(tt - (int64_t)b * a.N);
        const int fi = ti * kCovTile + fo, fj = tj * kCovTile + fo;
        yi = scaled_key(a, h, beta, b, j, fi) - mu[fi];
        yj = scaled_key(a, h, beta, b, j, fj) - mu[fj];
      }
      s_i[tk][fo] = yi;
      s_j[tk][fo] = yj;
    }
    __syncthreads();
#pragma unroll 4
    for (int tk = 0; tk < kCovTok; ++tk) {
      double xi[4], xj[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        xi[u] = s_i[tk][ri + u];
        xj[u] = s_j[tk][rj + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(xi[u], xj[v], acc[u][v]);
    }
    __syncthreads();
  }
  double* out = a.cov + (int64_t)hb * F * F;
  const double inv = 1.0 / (double)n;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      out[(int64_t)(ti * kCovTile + ri + u) * F + tj * kCovTile + rj + v] = acc[u][v] * inv;
}

hipError_t launch_tasq_stats(const TasqStatsArgs& a, hipStream_t s) {
  const int F = a.T_c * a.D;
  if (F % kCovTile || F > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tasq_mean_kernel, dim3(a.H * a.n_blk), dim3(F), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nt = F / kCovTile;
  hipLaunchKernelGGL(tasq_cov_kernel, dim3(nt * nt, a.H * a.n_blk), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace loopvq
