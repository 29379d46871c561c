// One step of the importance-weighted k-means that builds LoopVQ codebooks.
//
// LoopVQ review (arXiv 2611.05304), "codebook and calibration" (eq. 3): the
// codebook is trained offline by k-means in which each joint vector n is
// weighted by omega_n = ||dL/dz_n||^2; for a loop-axis joint vector the weight
// covers all T_c steps (section 3.1).  The assignment is the encode's exact
// argmin (loopvq_encode writes it); this file holds the update:
//   kmeans_accumulate_kernel: sums[r] += omega_n z_n, wsum[r] += omega_n over
//     the vectors assigned to codeword r, per (kv-head, block), in fp64;
//   kmeans_finalize_kernel: e_r = bf16_rne(sums[r] / wsum[r]) where wsum > 0.
// Joint coordinate u = i*T_c + m of chunk q is channel q*c + i at block step
// m (section 3.1 eq. 4); with the key pre-transform the vector is
// w[p(d')] * k[p(d')] / sigma (section 3.3), formed in fp64.
#include "common.h"
#include "kernels.h"

namespace loopvq {

namespace {

constexpr int kKmTok = 64;   // tokens per workgroup

// Round an fp64 value to the nearest bf16 (ties to even), exactly: the two
// candidates are the bf16 values around the value truncated toward zero.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  const uint32_t lo = __float_as_uint(__double2float_rz(v)) & 0xffff0000u;
  const uint32_t hi = lo + 0x10000u;   // next bf16 value away from zero
  const double dlo = fabs(v - (double)__uint_as_float(lo));
  const double dhi = fabs((double)__uint_as_float(hi) - v);
  if (dlo < dhi) return (uint16_t)(lo >> 16);
  if (dhi < dlo) return (uint16_t)(hi >> 16);
  return (uint16_t)(((lo >> 16) & 1u) ? hi >> 16 : lo >> 16);
}

}  // namespace

template <int G, bool TASQ>
__global__ __launch_bounds__(256) void kmeans_accumulate_kernel(KmeansArgs a) {
  __shared__ double s_acc[256 * (G + 1)];    // [K * G] sums, then [K] weights
  const int K = a.K, TC = a.T_c, C = G / TC, CPT = a.D / C;
  double* s_sum = s_acc;
  double* s_w = s_acc + K * G;
  const int tid = threadIdx.x;
  const int hb = blockIdx.y, h = hb / a.n_blk, beta = hb - h * a.n_blk;
  const int b = blockIdx.z;
  for (int e = tid; e < K * (G + 1); e += 256) s_acc[e] = 0.0;
  __syncthreads();

  const int j0 = blockIdx.x * kKmTok;
  const int ntok = min(kKmTok, a.N - j0);
  const int64_t row0 = ((int64_t)b * a.H + h) * a.n_blk + beta;
  for (int cl = tid; cl < ntok * CPT; cl += 256) {
    const int j = j0 + cl / CPT, q = cl - (cl / CPT) * CPT;
    const int r = a.idx[(row0 * a.N_cap + j) * CPT + q];
    if (r >= K) continue;                    // not a codeword of this codebook
    const double om = a.weight ? (double)a.weight[(row0 * a.N + j) * CPT + q] : 1.0;
    for (int u = 0; u < G; ++u) {
      const int i = u / TC, m = u - i * TC;
      const int t = beta * TC + m;
      const int dq = q * C + i;
      const uint16_t* xr = a.x + b * a.xs0 + h * a.xs1 + t * a.xs2 + (int64_t)j * a.xs3;
      double z;
      if constexpr (TASQ) {
        const int o = a.perm[h * a.D + dq] & (a.D - 1);
        const double sg = f16_bits_to_f64(a.sigma[((int64_t)b * a.sig_cap + j) * a.T + t]);
        z = ((double)a.w[h * a.D + o] * (double)bf16_to_f32(xr[o])) / sg;
      } else {
        z = (double)bf16_to_f32(xr[dq]);
      }
      atomicAdd(&s_sum[r * G + u], om * z);
    }
    atomicAdd(&s_w[r], om);
  }
  __syncthreads();
  double* gs = a.sums + (int64_t)hb * K * G;
  double* gw = a.wsum + (int64_t)hb * K;
  for (int e = tid; e < K * G; e += 256)
    if (s_sum[e] != 0.0) unsafeAtomicAdd(&gs[e], s_sum[e]);
  for (int e = tid; e < K; e += 256)
    if (s_w[e] != 0.0) unsafeAtomicAdd(&gw[e], s_w[e]);
}

__global__ __launch_bounds__(256) void kmeans_finalize_kernel(const double* __restrict__ sums,
                                                              const double* __restrict__ wsum,
                                                              uint16_t* __restrict__ cb, int64_t n, int G) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const double wt = wsum[e / G];
  if (wt > 0.0) cb[e] = f64_to_bf16_rne(sums[e] / wt);
}

template <int G>
static hipError_t km_launch(const KmeansArgs& a, int B, bool tasq, hipStream_t s) {
  const dim3 grid((a.N + kKmTok - 1) / kKmTok, a.H * a.n_blk, B);
  if (tasq)
    hipLaunchKernelGGL((kmeans_accumulate_kernel<G, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((kmeans_accumulate_kernel<G, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_kmeans_accumulate(const KmeansArgs& a, int B, bool tasq, hipStream_t s) {
  if (a.K > 256) return hipErrorInvalidValue;
  if (a.G == 16) return km_launch<16>(a, B, tasq, s);
  if (a.G == 32) return km_launch<32>(a, B, tasq, s);
  return hipErrorInvalidValue;
}

hipError_t launch_kmeans_finalize(const double* sums, const double* wsum, uint16_t* cb, int64_t n, int G,
                                  hipStream_t s) {
  hipLaunchKernelGGL(kmeans_finalize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, sums, wsum, cb,
                     n, G);
  return hipGetLastError();
}

// Importance weight of every joint vector (eq. 3): omega_n = ||dL/dz_n||^2,
// summed over the G coordinates of the vector, i.e. over the c channels of its
// chunk at each of the T_c steps of its block.  The gradient comes per cached
// element (dk for pre-RoPE keys, dv for values, as the precise-cache attention
// backward writes them).  With the keys' pre-transform z[d'] = w[p(d')]
// k[p(d')] / sigma, the chain rule gives dL/dz[d'] = dL/dk[p(d')] sigma /
// w[p(d')] (sigma is a stored constant, not part of the code).  One thread per
// (batch, kv-head, block, token, chunk); blockIdx.y picks keys or values.
__global__ __launch_bounds__(256) void fisher_kernel(FisherArgs a) {
  const int kv = blockIdx.y;
  const int C = a.G / a.T_c, CPT = a.D / C;
  const int64_t n = (int64_t)a.B * a.H * a.n_blk * a.N * CPT;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  int64_t r = e;
  const int q = (int)(r % CPT);
  r /= CPT;
  const int j = (int)(r % a.N);
  r /= a.N;
  const int beta = (int)(r % a.n_blk);
  r /= a.n_blk;
  const int h = (int)(r % a.H);
  const int b = (int)(r / a.H);
  const bool tasq = kv == 0 && a.perm != nullptr;
  const float* g = kv == 0 ? a.dk : a.dv;
  double acc = 0.0;
  for (int m = 0; m < a.T_c; ++m) {
    const int t = beta * a.T_c + m;
    const float* row = g + ((((int64_t)b * a.H + h) * a.T + t) * a.N_x + j) * a.D;
    double sg = 1.0;
    if (tasq) sg = f16_bits_to_f64(a.sigma[((int64_t)b * a.sig_cap + j) * a.T + t]);
    for (int i = 0; i < C; ++i) {
      const int dp = q * C + i;
      double v;
      if (tasq) {
        const int o = a.perm[h * a.D + dp] & (a.D - 1);
        v = (double)row[o] * sg / (double)a.w[h * a.D + o];
      } else {
        v = (double)row[dp];
      }
      acc += v * v;
    }
  }
  (kv == 0 ? a.wk : a.wv)[e] = (float)acc;
}

hipError_t launch_fisher(const FisherArgs& a, hipStream_t s) {
  const int C = a.G / a.T_c;
  const int64_t n = (int64_t)a.B * a.H * a.n_blk * a.N * (a.D / C);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fisher_kernel, dim3((unsigned)((n + 255) / 256), 2), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace loopvq
