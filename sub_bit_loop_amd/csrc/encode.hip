// LoopVQ encode: nearest codeword of every loop-axis joint vector.
//
// LoopVQ review (arXiv 2611.05304), section "terms" eq. (2): a(z) =
// argmin_r ||z - e_r||^2; section 3.1 eq. (4): coordinate i*T_c + m of the
// joint vector is channel q*c + i of block step m; section 3.4 step 2: the
// distances to every codebook entry are a dense matrix product.
//
// Each workgroup owns one (batch, kv-head, block) and 64 tokens.  The block's
// codebook is staged in LDS as -2*e (bf16, exact) with ||e||^2 (fp32); a wave
// takes 32 codes at a time and evaluates
//     dt_r = ||e_r||^2 - 2 z.e_r    (= ||z - e_r||^2 - ||z||^2)
// for 32 codewords per v_mfma_f32_32x32x16_bf16 (codewords on M, codes on N,
// ||e||^2 preloaded in the accumulator), keeping a per-lane best/second-best.
// A code whose two best screened values lie within twice the fp32 error bound
// is re-scored exactly in fp64 (direct form, lowest index on ties), so the
// written index is the exact argmin.
#include "common.h"
#include "kernels.h"

namespace loopvq {

// fp64 -> fp16 bits, round to nearest even, for non-negative finite v.
__device__ __forceinline__ uint16_t f64_to_f16_rne(double v) {
  _Float16 h0 = (_Float16)(float)v;
  uint16_t b0;
  __builtin_memcpy(&b0, &h0, 2);
  uint16_t best = b0;
  double bestd = fabs(v - f16_bits_to_f64(b0));
  for (int k = -1; k <= 1; k += 2) {
    int c = (int)b0 + k;
    if (c < 0 || c >= 0x7c00) continue;
    double d = fabs(v - f16_bits_to_f64((uint16_t)c));
    if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) != 0)) {
      best = (uint16_t)c;
      bestd = d;
    }
  }
  return best;
}

// Per-(token, step) RMS of the layer's raw keys over all heads and channels,
// in fp64, rounded to fp16 (review section 3.3 / appendix B).  One wave per
// token; lane l covers channels 2l, 2l+1 of every head.
__global__ __launch_bounds__(256) void sigma_kernel(SigmaArgs a) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (j >= a.N) return;
  for (int t = 0; t < a.T; ++t) {
    double s = 0.0;
    for (int h = 0; h < a.H; ++h) {
      const uint16_t* row = a.x + b * a.xs0 + h * a.xs1 + t * a.xs2 + (int64_t)j * a.xs3;
      uint32_t wv = *reinterpret_cast<const uint32_t*>(row + 2 * lane);
      double lo = bf16lo(wv), hi = bf16hi(wv);
      s += lo * lo + hi * hi;
    }
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    if (lane == 0) {
      double sig = sqrt(s / (double)(a.H * 128));
      a.sigma[((int64_t)b * a.sig_cap + a.tok0 + j) * a.T + t] = f64_to_f16_rne(sig);
    }
  }
}

template <int G, int TC, bool TASQ>
__global__ __launch_bounds__(kEncodeThreads) void encode_kernel(EncodeArgs a) {
  constexpr int D = 128;
  constexpr int C = G / TC;        // channels per step per code
  constexpr int CPT = D / C;       // codes per token
  constexpr int KK = G / 16;       // MFMA k-chunks of 16
  __shared__ __attribute__((aligned(16))) uint16_t s_cb[256 * G];
  __shared__ __attribute__((aligned(16))) float s_nrm[256];
  __shared__ float s_wmax[kEncodeThreads / kWave];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hb = blockIdx.y;
  const int h = hb / a.n_blk, beta = hb - h * a.n_blk;
  const int b = blockIdx.z;
  const uint16_t* cb = a.cb + (int64_t)hb * a.K * G;

  for (int e = tid; e < 256 * G; e += kEncodeThreads) {
    uint16_t v = 0;
    if (e < a.K * G) v = (uint16_t)f32_to_bf16_rne(-2.f * bf16_to_f32(cb[e]));
    s_cb[e] = v;
  }
  float nmax = 0.f;
  {
    const int r = tid;
    float nrm = INFINITY;
    if (r < a.K) {
      float s = 0.f;
      for (int u = 0; u < G; ++u) {
        float f = bf16_to_f32(cb[r * G + u]);
        s = fmaf(f, f, s);
      }
      nrm = s;
      nmax = s;
    }
    s_nrm[r] = nrm;
  }
  for (int off = 32; off >= 1; off >>= 1) nmax = fmaxf(nmax, __shfl_xor(nmax, off));
  if (lane == 0) s_wmax[wave] = nmax;
  __syncthreads();
  const float emax = fmaxf(fmaxf(s_wmax[0], s_wmax[1]), fmaxf(s_wmax[2], s_wmax[3]));

  const int j0 = blockIdx.x * kEncodeTokens;
  const int j1 = min(j0 + kEncodeTokens, a.N);
  const int ncodes = (j1 - j0) * CPT;
  const int ngroups = (ncodes + 31) >> 5;
  const int n = lane & 31, hh = lane >> 5;
  const uint16_t* xbase = a.x + b * a.xs0 + h * a.xs1 + (int64_t)(beta * TC) * a.xs2;
  uint8_t* ibase = a.idx + (((int64_t)b * a.H + h) * a.n_blk + beta) * (int64_t)a.N_cap * CPT +
                   (int64_t)(a.tok0 + j0) * CPT;
  const float* wh = TASQ ? a.w + h * D : nullptr;
  const int16_t* ph = TASQ ? a.perm + h * D : nullptr;
  const uint16_t* sgb = TASQ ? a.sigma + ((int64_t)b * a.sig_cap + a.tok0) * a.T + beta * TC : nullptr;

  for (int grp = wave; grp < ngroups; grp += kEncodeThreads / kWave) {
    const int g = grp * 32 + n;
    const bool valid = g < ncodes;
    const int gg = valid ? g : ncodes - 1;
    const int jl = gg / CPT, q = gg - jl * CPT;
    const int j = j0 + jl;
    const uint16_t* xr = xbase + (int64_t)j * a.xs3;

    // B operand: this lane's 8 joint coordinates per k-chunk.
    bf16x8_t bz[KK];
    bf16x8_t bzlo[KK];
    float zz = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int u = 16 * kk + 8 * hh + e;
        const int i = u / TC, m = u - (u / TC) * TC;
        const int d = q * C + i;
        if constexpr (!TASQ) {
          uint16_t v = xr[m * a.xs2 + d];
          float f = bf16_to_f32(v);
          zz = fmaf(f, f, zz);
          bz[kk][e] = __builtin_bit_cast(__bf16, v);
        } else {
          const int o = ph[d] & (D - 1);
          float kv = bf16_to_f32(xr[m * a.xs2 + o]);
          _Float16 sh;
          uint16_t sb = sgb[(int64_t)j * a.T + m];
          __builtin_memcpy(&sh, &sb, 2);
          float zf = (wh[o] * kv) / (float)sh;
          uint32_t hb16 = f32_to_bf16_rne(zf);
          uint32_t lb16 = f32_to_bf16_rne(zf - bf16_to_f32(hb16));
          zz = fmaf(zf, zf, zz);
          bz[kk][e] = __builtin_bit_cast(__bf16, (uint16_t)hb16);
          bzlo[kk][e] = __builtin_bit_cast(__bf16, (uint16_t)lb16);
        }
      }
    }

    float b1 = INFINITY, b2 = INFINITY;
    int i1 = 0;
#pragma unroll 1
    for (int t = 0; t < 8; ++t) {
      f32x16_t acc;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        f32x4_t nv = *reinterpret_cast<const f32x4_t*>(&s_nrm[32 * t + 8 * v + 4 * hh]);
        acc[4 * v + 0] = nv[0];
        acc[4 * v + 1] = nv[1];
        acc[4 * v + 2] = nv[2];
        acc[4 * v + 3] = nv[3];
      }
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&s_cb[(32 * t + n) * G + 16 * kk + 8 * hh]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bz[kk], acc, 0, 0, 0);
        if constexpr (TASQ) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bzlo[kk], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float v = acc[i];
        const int r = 32 * t + 8 * (i >> 2) + 4 * hh + (i & 3);
        b2 = fminf(b2, fmaxf(b1, v));
        if (v < b1) {
          b1 = v;
          i1 = r;
        }
      }
    }
    // Combine the two half-waves (lanes n and n+32 hold different codewords).
    const float ob1 = __shfl_xor(b1, 32), ob2 = __shfl_xor(b2, 32);
    const int oi1 = __shfl_xor(i1, 32);
    zz += __shfl_xor(zz, 32);
    float nb1;
    int ni1;
    if (ob1 < b1 || (ob1 == b1 && oi1 < i1)) {
      nb1 = ob1;
      ni1 = oi1;
    } else {
      nb1 = b1;
      ni1 = i1;
    }
    const float nb2 = fminf(fmaxf(b1, ob1), fminf(b2, ob2));
    if (hh == 0 && valid) {
      // Screening error bound on dt (fp32 sums of G+1 terms plus the norm).
      float eps = (float)(2 * G + 2) * 5.9604645e-08f * (2.f * emax + zz);
      if constexpr (TASQ) eps = 2.f * eps + 1.5258789e-05f * (zz + emax);
      int res = ni1;
      if (!(nb2 > nb1 + 2.f * eps)) {
        // Exact re-score in fp64, direct form, lowest index wins.
        double zd[G];
#pragma unroll
        for (int u = 0; u < G; ++u) {
          const int i = u / TC, m = u - (u / TC) * TC;
          const int d = q * C + i;
          if constexpr (!TASQ) {
            zd[u] = (double)bf16_to_f32(xr[m * a.xs2 + d]);
          } else {
            const int o = ph[d] & (D - 1);
            double kv = (double)bf16_to_f32(xr[m * a.xs2 + o]);
            double sg = f16_bits_to_f64(sgb[(int64_t)j * a.T + m]);
            zd[u] = ((double)wh[o] * kv) / sg;
          }
        }
        double best = INFINITY;
        int bi = 0;
        for (int r = 0; r < a.K; ++r) {
          double dist = 0.0;
#pragma unroll
          for (int u = 0; u < G; ++u) {
            double e = -0.5 * (double)bf16_to_f32(s_cb[r * G + u]);
            double df = zd[u] - e;
            dist += df * df;
          }
          if (dist < best) {
            best = dist;
            bi = r;
          }
        }
        res = bi;
      }
      ibase[g] = (uint8_t)res;
    }
  }
}

template <int G, int TC>
static hipError_t enc_launch(bool tasq, const EncodeArgs& a, int B, hipStream_t s) {
  dim3 grid((a.N + kEncodeTokens - 1) / kEncodeTokens, a.H * a.n_blk, B);
  if (tasq)
    hipLaunchKernelGGL((encode_kernel<G, TC, true>), grid, dim3(kEncodeThreads), 0, s, a);
  else
    hipLaunchKernelGGL((encode_kernel<G, TC, false>), grid, dim3(kEncodeThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_encode(int G, int TC, bool tasq, const EncodeArgs& a, int B, hipStream_t s) {
  if (G == 16) {
    switch (TC) {
      case 1: return enc_launch<16, 1>(tasq, a, B, s);
      case 2: return enc_launch<16, 2>(tasq, a, B, s);
      case 4: return enc_launch<16, 4>(tasq, a, B, s);
      case 8: return enc_launch<16, 8>(tasq, a, B, s);
    }
  } else if (G == 32) {
    switch (TC) {
      case 1: return enc_launch<32, 1>(tasq, a, B, s);
      case 2: return enc_launch<32, 2>(tasq, a, B, s);
      case 4: return enc_launch<32, 4>(tasq, a, B, s);
      case 8: return enc_launch<32, 8>(tasq, a, B, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_sigma(const SigmaArgs& a, int B, hipStream_t s) {
  dim3 grid((a.N + 3) / 4, B);
  hipLaunchKernelGGL(sigma_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace loopvq
