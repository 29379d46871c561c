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

// Split an fp32 value into three bf16 terms whose sum is exact (RNE splits).
__device__ __forceinline__ void split3(float x, uint16_t& h, uint16_t& m, uint16_t& l) {
  uint32_t a = f32_to_bf16_rne(x);
  float r1 = x - bf16_to_f32(a);
  uint32_t b = f32_to_bf16_rne(r1);
  float r2 = r1 - bf16_to_f32(b);
  h = (uint16_t)a;
  m = (uint16_t)b;
  l = (uint16_t)f32_to_bf16_rne(r2);
}

// bf16 bits of the smallest bf16 >= x (x > 0 finite).
__device__ __forceinline__ uint16_t bf16_ceil(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t hi = u >> 16;
  if (u & 0xffffu) ++hi;
  return (uint16_t)hi;
}

template <int G, int TC, bool TASQ>
__global__ __launch_bounds__(kEncodeThreads) void encode_kernel(EncodeArgs a) {
  constexpr int D = 128;
  constexpr int C = G / TC;        // channels per step per code
  constexpr int CPT = D / C;       // codes per token
  constexpr int KK = G / 16;       // MFMA k-chunks of 16
  // Per codebook row: -2*e (G bf16) and the norm row [nh, nm, nl, 1, 1, 1, 1, 0].
  __shared__ __attribute__((aligned(16))) uint16_t s_cb[256 * G];
  __shared__ __attribute__((aligned(16))) uint16_t s_nb[256 * 8];
  __shared__ float s_wmax[kEncodeThreads / kWave];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hb = blockIdx.y;
  const int h = hb / a.n_blk, beta = hb - h * a.n_blk;
  const int b = blockIdx.z;
  const uint16_t* cb = a.cb + (int64_t)hb * a.K * G;

  float nmax = 0.f;
  {
    const int r = tid;   // one codebook row per thread
    uint16_t nh = 0, nm = 0, nl = 0;
    uint16_t one = 0;
    if (r < a.K) {
      double s = 0.0;
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const float f = bf16_to_f32(cb[r * G + u]);
        s += (double)f * (double)f;
        s_cb[r * G + u] = (uint16_t)f32_to_bf16_rne(-2.f * f);
      }
      const float nf = (float)s;
      split3(nf, nh, nm, nl);
      nmax = nf;
      one = 0x3f80;
    } else {
      // Padding rows never win: a huge norm, zero codeword.
#pragma unroll
      for (int u = 0; u < G; ++u) s_cb[r * G + u] = 0;
      nh = 0x7f00;   // 2^127
    }
    uint16_t* nb = s_nb + r * 8;
    nb[0] = nh; nb[1] = nm; nb[2] = nl; nb[3] = one; nb[4] = one; nb[5] = one; nb[6] = 0x3f80; nb[7] = 0;
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
  const uint32_t kmask = 0xffffff00u;   // the low byte carries the lane-local candidate number

  for (int grp = wave; grp < ngroups; grp += kEncodeThreads / kWave) {
    const int g = grp * 32 + n;
    const bool valid = g < ncodes;
    const int gg = valid ? g : ncodes - 1;
    const int jl = gg / CPT, q = gg - jl * CPT;
    const int j = j0 + jl;
    const uint16_t* xr = xbase + (int64_t)j * a.xs3;

    // B operand: this lane's 8 joint coordinates per k-chunk (code n, coordinates 16kk+8hh..+7).
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
          const uint16_t v = xr[m * a.xs2 + d];
          const float f = bf16_to_f32(v);
          zz = fmaf(f, f, zz);
          bz[kk][e] = __builtin_bit_cast(__bf16, v);
        } else {
          const int o = ph[d] & (D - 1);
          const float kv = bf16_to_f32(xr[m * a.xs2 + o]);
          _Float16 sh;
          const uint16_t sb = sgb[(int64_t)j * a.T + m];
          __builtin_memcpy(&sh, &sb, 2);
          const float zf = (wh[o] * kv) / (float)sh;
          const uint32_t hb16 = f32_to_bf16_rne(zf);
          const uint32_t lb16 = f32_to_bf16_rne(zf - bf16_to_f32(hb16));
          zz = fmaf(zf, zf, zz);
          bz[kk][e] = __builtin_bit_cast(__bf16, (uint16_t)hb16);
          bzlo[kk][e] = __builtin_bit_cast(__bf16, (uint16_t)lb16);
        }
      }
    }
    zz += __shfl_xor(zz, 32);   // ||z||^2 of code n (both halves)
    // Error bound of the screened distance, and a margin that keeps every
    // screened value positive so its bit pattern orders like the value.
    float eps = (float)(G + 24) * 5.9604645e-08f * (2.f * emax + 2.f * zz);
    if constexpr (TASQ) eps = 2.f * eps + 3.0517578e-05f * (zz + emax);
    const uint16_t beta_b = bf16_ceil(2.f * eps + 1e-30f);
    bf16x8_t bn;
    {
      uint16_t zh, zm, zl;
      split3(zz, zh, zm, zl);
      const uint16_t one = hh == 0 ? 0x3f80 : 0;
      bn[0] = __builtin_bit_cast(__bf16, one);
      bn[1] = __builtin_bit_cast(__bf16, one);
      bn[2] = __builtin_bit_cast(__bf16, one);
      bn[3] = __builtin_bit_cast(__bf16, (uint16_t)(hh == 0 ? zh : 0));
      bn[4] = __builtin_bit_cast(__bf16, (uint16_t)(hh == 0 ? zm : 0));
      bn[5] = __builtin_bit_cast(__bf16, (uint16_t)(hh == 0 ? zl : 0));
      bn[6] = __builtin_bit_cast(__bf16, (uint16_t)(hh == 0 ? beta_b : 0));
      bn[7] = __builtin_bit_cast(__bf16, (uint16_t)0);
    }

    // Screening: every value is ||z - e_r||^2 + margin (fp32 MFMA); the key
    // replaces the low mantissa byte with the lane-local candidate number.
    // Keys are positive finite floats whose low byte is the candidate number,
    // so float min / median order them exactly like the screened values.
    float k1 = INFINITY, k2 = INFINITY;
#pragma unroll 2
    for (int t = 0; t < 8; ++t) {
      f32x16_t acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const bf16x8_t an = *reinterpret_cast<const bf16x8_t*>(&s_nb[(32 * t + n) * 8 + 0]);
      bf16x8_t anz;
      if (hh == 0) anz = an; else anz = bf16x8_t{};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(anz, bn, acc, 0, 0, 0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&s_cb[(32 * t + n) * G + 16 * kk + 8 * hh]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bz[kk], acc, 0, 0, 0);
        if constexpr (TASQ) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bzlo[kk], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float key = __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(acc[i]), (uint32_t)(16 * t + i), 0x07060500u));
        k2 = __builtin_amdgcn_fmed3f(k1, k2, key);
        k1 = fminf(k1, key);
      }
    }
    // Merge the two half-waves (lanes n and n+32 screen different codewords).
    const uint32_t uk1 = __float_as_uint(k1), uk2 = __float_as_uint(k2);
    const uint32_t ok1 = __shfl_xor(uk1, 32), ok2 = __shfl_xor(uk2, 32);
    const float v1 = __uint_as_float(uk1 & kmask), ov1 = __uint_as_float(ok1 & kmask);
    const bool mine = v1 < ov1 || (v1 == ov1 && hh == 0);
    const uint32_t wkey = mine ? uk1 : ok1;
    const int whalf = mine ? hh : hh ^ 1;
    const float t1 = __uint_as_float(wkey & kmask);
    // second smallest screened value over both halves
    const float s_own2 = __uint_as_float(uk2 & kmask), s_oth2 = __uint_as_float(ok2 & kmask);
    const float t2 = mine ? fminf(s_own2, ov1) : fminf(s_oth2, v1);
    const float thr = t1 * (1.f + 6.1035156e-05f) + 2.f * eps;
    const bool tie = valid && !(t2 > thr);
    const int loc = (int)(wkey & 0xffu);
    int res = 32 * (loc >> 4) + 8 * ((loc & 15) >> 2) + 4 * whalf + (loc & 3);

    if (__builtin_expect(__ballot(tie) != 0, 0)) {
      // Rare path: re-screen and score every candidate inside the band exactly
      // in fp64 (direct form); lowest index wins exact ties.
      double zd[G];
      if (tie) {
#pragma unroll
        for (int u = 0; u < G; ++u) {
          const int i = u / TC, m = u - (u / TC) * TC;
          const int d = q * C + i;
          if constexpr (!TASQ) {
            zd[u] = (double)bf16_to_f32(xr[m * a.xs2 + d]);
          } else {
            const int o = ph[d] & (D - 1);
            const double kv = (double)bf16_to_f32(xr[m * a.xs2 + o]);
            const double sg = f16_bits_to_f64(sgb[(int64_t)j * a.T + m]);
            zd[u] = ((double)wh[o] * kv) / sg;
          }
        }
      }
      const float lim = tie ? thr : -1.f;
      double best = INFINITY;
      int bi = 0x7fffffff;
#pragma unroll 1
      for (int t = 0; t < 8; ++t) {
        f32x16_t acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const bf16x8_t an = *reinterpret_cast<const bf16x8_t*>(&s_nb[(32 * t + n) * 8 + 0]);
        bf16x8_t anz;
        if (hh == 0) anz = an; else anz = bf16x8_t{};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(anz, bn, acc, 0, 0, 0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&s_cb[(32 * t + n) * G + 16 * kk + 8 * hh]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bz[kk], acc, 0, 0, 0);
          if constexpr (TASQ) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bzlo[kk], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float tv = __uint_as_float(__float_as_uint(acc[i]) & kmask);
          if (tv <= lim) {
            const int r = 32 * t + 8 * (i >> 2) + 4 * hh + (i & 3);
            double dist = 0.0;
            for (int u = 0; u < G; ++u) {
              const double e = -0.5 * (double)bf16_to_f32(s_cb[r * G + u]);
              const double df = zd[u] - e;
              dist += df * df;
            }
            if (r < a.K && (dist < best || (dist == best && r < bi))) {
              best = dist;
              bi = r;
            }
          }
        }
      }
      // combine the halves: smallest distance, then lowest index
      const double obest = __shfl_xor(best, 32);
      const int obi = __shfl_xor(bi, 32);
      if (obest < best || (obest == best && obi < bi)) {
        best = obest;
        bi = obi;
      }
      if (tie) res = bi;
    }
    if (hh == 0 && valid) ibase[g] = (uint8_t)res;
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
