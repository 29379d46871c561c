// LoopVQ encode: nearest codeword of every loop-axis joint vector.
//
// LoopVQ review (arXiv 2611.05304), section "terms" eq. (2): a(z) =
// argmin_r ||z - e_r||^2; section 3.1 eq. (4): coordinate i*T_c + m of the
// joint vector is channel q*c + i of block step m; section 3.4 step 2: the
// distances to every codebook entry are a dense matrix product.
//
// Each workgroup owns one (batch, kv-head, block) and 128 tokens.  The
// block's codebook is staged once as -2*e (bf16, exact) with ||e||^2 split
// into three bf16 terms; each wave then keeps the A operands of all 8
// codeword tiles in registers.  A wave takes 32 codes at a time (two 8-byte
// loads per lane: joint coordinates are taken in step-major order, so each
// lane reads contiguous channels of two steps) and evaluates
//     s_r = ||e_r||^2 + u - 2 z.e_r    (u ~ ||z||^2, common to all r)
// for 32 codewords per tile: a v_mfma_f32_32x32x8 for the norm terms and a
// v_mfma_f32_32x32x16_bf16 for the products (codewords on M, codes on N).
// At G = 16 each lane reduces every four consecutive codewords to their
// smallest screened value and keys only that value (group number in the low
// mantissa byte); the winning group is scored again in fp32 after the
// screening.  At G = 32 every screened value gets a key (candidate number in
// the low byte).  Pre-transformed keys enter the products as two bf16 terms
// (hi + lo) of their fp32 value.  Best and second-best keys cost one
// min3, one med3 and one min per two keys.  A code whose two best values lie
// within the fp32 error band is re-scored exactly in fp64 (direct form,
// lowest index on ties), so the written index is the exact argmin.
#include "common.h"
#include "kernels.h"

namespace loopvq {

// Per-(token, step) RMS of the layer's raw keys over all heads and channels,
// in fp64, rounded to fp16 (review section 3.3 / appendix B).  One wave per
// token; a 16-byte load per lane covers four heads at once: lane l reads
// channels 8(l % 16) .. +7 of heads l/16, l/16 + 4, ...  (rows are 16-byte
// aligned: the entry point requires it).
__global__ __launch_bounds__(256) void sigma_kernel(SigmaArgs a) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = blockIdx.y;
  if (j >= a.N) return;
  const int h0 = lane >> 4, c8 = 8 * (lane & 15);
  for (int t = 0; t < a.T; ++t) {
    double s = 0.0;
    for (int h = h0; h < a.H; h += 4) {
      const uint16_t* row = a.x + b * a.xs0 + h * a.xs1 + t * a.xs2 + (int64_t)j * a.xs3;
      const uint4 w = *reinterpret_cast<const uint4*>(row + c8);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double lo = bf16lo(ws[k]), hi = bf16hi(ws[k]);
        s += lo * lo + hi * hi;
      }
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

template <int G, int TC, bool TASQ>
__global__ __launch_bounds__(kEncodeThreads, (G == 16 && !TASQ) ? 4 : 1) void encode_kernel(EncodeArgs a) {
  constexpr int D = 128;
  constexpr int C = G / TC;          // channels per step per code
  constexpr int CPT = D / C;         // codes per token
  constexpr int LOG_CPT = __builtin_ctz(CPT);
  constexpr int KK = G / 16;         // MFMA k-chunks of 16
  constexpr int CW = C < 8 ? C : 8;  // contiguous channels per load
  constexpr int NL = 8 / CW;         // loads per 8-position slot
  static_assert(C >= 2 && (CPT & (CPT - 1)) == 0, "unsupported code shape");
  // Selection per group of four candidates (G = 16) or per candidate.  At
  // G = 32 the matrix cores take 1.5x longer per group of codes and the
  // per-candidate form measured faster.
  constexpr bool kGroups = G == 16;
  // Per codebook row: -2*e in step-major order (G bf16) and the norm row
  // [nh, nm, nl, 1] (||e||^2 split into three bf16 terms).  With group
  // selection, rows are stored in blocks of four with 16 bytes of padding
  // after each block, so that the 16-byte reads of the rows 4g .. 4g+3 of 64
  // random blocks g (one per lane) spread over all LDS banks instead of two
  // 16-byte slots.
  constexpr int kCbBlock = kGroups ? 4 * G + 8 : 4 * G;
  __shared__ __attribute__((aligned(16))) uint16_t s_cb[64 * kCbBlock];
  auto cbrow = [](int r) { return (r >> 2) * kCbBlock + (r & 3) * G; };
  __shared__ __attribute__((aligned(16))) uint16_t s_nb[256 * 4];
  // ||e||^2 in fp32 (the value nh + nm + nl), read when a group of four
  // candidates is scored again after screening.
  __shared__ __attribute__((aligned(16))) float s_nf[256];
  // Codes of this workgroup (token * CPT + chunk) whose two best screened
  // values lie within the exactness band; they are scored exactly after the
  // screening loop, one code per wave at a time.
  __shared__ uint16_t s_tq[kEncodeTokens * CPT];
  __shared__ int s_tqn;
  // Pre-transformed keys with CPT <= 32: the rows of a group's tokens (all
  // T_c steps of its 32 / CPT tokens, 64 G bytes) are read with 16-byte loads
  // (G / 16 per lane) into the wave's staging area, and every lane picks its
  // positions' raw channels from there.
  constexpr bool kStaged = TASQ && CPT <= 32;
  constexpr int kStageU4 = 4 * G;    // uint4 per wave
  __shared__ __attribute__((aligned(16))) uint4 s_stage[kStaged ? (kEncodeThreads / kWave) * kStageU4 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hb = blockIdx.y;
  const int h = hb / a.n_blk, beta = hb - h * a.n_blk;
  const int b = blockIdx.z;
  const uint16_t* cb = a.cb + (int64_t)hb * a.K * G;

  {
    const int r = tid;   // one codebook row per thread
    uint16_t nh = 0, nm = 0, nl = 0, one = 0;
    if (r < a.K) {
      double s = 0.0;
#pragma unroll
      for (int p = 0; p < G; ++p) {
        // position p = m*C + i holds joint coordinate i*T_c + m
        const float f = bf16_to_f32(cb[r * G + (p % C) * TC + p / C]);
        s += (double)f * (double)f;
        s_cb[cbrow(r) + p] = (uint16_t)f32_to_bf16_rne(-2.f * f);
      }
      const float nf = (float)s;
      split3(nf, nh, nm, nl);
      s_nf[r] = nf;
      one = 0x3f80;
    } else {
      // Padding rows never win: a huge norm, zero codeword.
#pragma unroll
      for (int p = 0; p < G; ++p) s_cb[cbrow(r) + p] = 0;
      nh = 0x7f00;   // 2^127
      s_nf[r] = 0x1p127f;
    }
    uint16_t* nb = s_nb + r * 4;
    nb[0] = nh; nb[1] = nm; nb[2] = nl; nb[3] = one;
  }
  if (tid == 0) s_tqn = 0;
  __syncthreads();

  const int n = lane & 31, hh = lane >> 5;
  // The A operands of all 8 codeword tiles stay in registers: row n of tile
  // t is codeword 32t + n; this half-wave holds positions 16kk + 8hh .. +7.
  // The norm rows are the A operand of a 32x32x8 product whose k = 4..7
  // half (second half-wave) meets zeros in B.
  s16x4_t an[8];
  bf16x8_t av[8][KK];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    an[t] = *reinterpret_cast<const s16x4_t*>(&s_nb[(32 * t + n) * 4]);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      av[t][kk] = *reinterpret_cast<const bf16x8_t*>(&s_cb[cbrow(32 * t + n) + 16 * kk + 8 * hh]);
  }

  const int j0 = blockIdx.x * kEncodeTokens;
  const int j1 = min(j0 + kEncodeTokens, a.N);
  const int ncodes = (j1 - j0) * CPT;
  const int ngroups = __builtin_amdgcn_readfirstlane((ncodes + 31) >> 5);
  const int64_t xs2 = a.xs2, xs3 = a.xs3;
  const uint16_t* xbase = a.x + b * a.xs0 + h * a.xs1 + (int64_t)(beta * TC) * xs2 + (int64_t)j0 * xs3;
  uint8_t* ibase = a.idx + (((int64_t)b * a.H + h) * a.n_blk + beta) * (int64_t)a.N_cap * CPT +
                   (int64_t)(a.tok0 + j0) * CPT;
  const float* wh = TASQ ? a.w + h * D : nullptr;
  const int16_t* ph = TASQ ? a.perm + h * D : nullptr;
  const uint16_t* sgb = TASQ ? a.sigma + ((int64_t)b * a.sig_cap + a.tok0 + j0) * a.T + beta * TC : nullptr;
  const uint32_t kmask = 0xffffff00u;   // the low byte carries the lane-local candidate number

  // Lane-constant part of the load address: slot s = 2kk + hh covers
  // positions 8s .. 8s+7, i.e. steps 8s/C .. and channels (8s % C) ...
  // With CPT >= 32 a group of 32 codes lies in one token (chunks n + a
  // group-uniform offset); otherwise it spans 32/CPT tokens.
  const int ntok = j1 - j0;
  int64_t loff[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    const int p0 = 8 * (2 * kk + hh);
    loff[kk] = (int64_t)(p0 / C) * xs2 + (p0 % C) + (CPT >= 32 ? n * C : (n & (CPT - 1)) * C);
  }
  // token (relative to j0) and chunk of this lane's code in group grp
  auto code_pos = [&](int grp, int& jl, int& q) {
    const int g0 = grp * 32;
    if constexpr (CPT >= 32) {
      jl = g0 >> LOG_CPT;
      q = (g0 & (CPT - 1)) + n;
    } else {
      jl = min((g0 >> LOG_CPT) + (n >> LOG_CPT), ntok - 1);
      q = n & (CPT - 1);
    }
  };

  // Pre-transformed keys: this lane's code is always chunk n mod CPT of its
  // token, so the raw channel p(d) and weight w[p(d)] of each of its joint
  // positions are lane constants; tof holds the element's place in the
  // staging area (row (token in group) * T_c + step, then the raw channel).
  int tof[TASQ ? KK : 1][8];
  float twt[TASQ ? KK : 1][8];
  if constexpr (kStaged) {
    const int tk = CPT < 32 ? (n >> LOG_CPT) : 0;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int p = 16 * kk + 8 * hh + e;
        const int o = ph[(n & (CPT - 1)) * C + (p % C)] & (D - 1);
        tof[kk][e] = (tk * TC + p / C) * D + o;
        twt[kk][e] = wh[o];
      }
  }

  // Loads the joint vectors of group grp: code g = 32*grp + n is token
  // g / CPT, chunk g % CPT.
  auto fetch = [&](int grp, bf16x8_t (&zh)[KK]) {
    int jl, q;
    code_pos(grp, jl, q);
    // group-uniform part of the address (the lane part is in loff)
    const uint16_t* xr = xbase + (int64_t)jl * xs3 + (CPT >= 32 ? (q - n) * C : 0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const uint16_t* pz = xr + loff[kk];
      if constexpr (CW == 8) {
        zh[kk] = *reinterpret_cast<const bf16x8_t*>(pz);
      } else {
        uint32_t w[4];
#pragma unroll
        for (int l = 0; l < NL; ++l) {
          if constexpr (CW == 4) {
            const uint2 v = *reinterpret_cast<const uint2*>(pz + l * xs2);
            w[2 * l] = v.x;
            w[2 * l + 1] = v.y;
          } else {
            w[l] = *reinterpret_cast<const uint32_t*>(pz + l * xs2);
          }
        }
        zh[kk] = __builtin_bit_cast(bf16x8_t, (uint4){w[0], w[1], w[2], w[3]});
      }
    }
  };
  // Pre-transformed keys, in two parts so that the loads of the next group
  // are in flight while the current one is screened: the raw bf16 bits of
  // k[p(d)] (through the staging area when CPT <= 32, else one 2-byte load
  // per position) and the fp16 bits of sigma for each joint position of the lane,
  // then z = w[p(d)] * k[p(d)] / sigma split into two bf16 terms hi + lo
  // (the residual is exact in fp32, the sum is within 2^-16 |z|; the band
  // below covers the split, near ties are re-scored from the inputs in
  // fp64).  Sigma is read once per step of the lane's positions and its
  // reciprocal taken once.
  // raw channel of position 16kk + 8hh + e of chunk q (c = 2, where the
  // lane's chunk changes between groups and the rows are not staged)
  auto raw_channel = [&](int kk, int e, int q) { return ph[q * C + ((16 * kk + 8 * hh + e) % C)] & (D - 1); };
  // positions 16kk + 8hh + e of slot kk cover NS steps: step
  // (16kk + 8hh) / C + e / CW
  constexpr int NS = 8 / CW;
  // staged form: 16-byte chunk lane + 64u of the group's rows (row = token
  // in group * T_c + step, 16 chunks of 8 channels per row) and sigma
  uint4 stg[kStaged ? KK : 1];
  auto fetch_stage = [&](int grp, uint32_t (&rs)[KK][NS]) {
    int jl, q;
    code_pos(grp, jl, q);
    const int jl0 = (grp * 32) >> LOG_CPT;
#pragma unroll
    for (int u = 0; u < KK; ++u) {
      const int c = lane + 64 * u, r = c >> 4;
      const int tok = min(jl0 + r / TC, ntok - 1);
      stg[u] = *reinterpret_cast<const uint4*>(xbase + (int64_t)tok * xs3 + (int64_t)(r % TC) * xs2 + 8 * (c & 15));
    }
    const uint16_t* sg = sgb + (int64_t)jl * a.T;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int l = 0; l < NS; ++l) rs[kk][l] = sg[(16 * kk + 8 * hh) / C + l];
  };
  // the staged rows through this wave's LDS area into the lane's raw key
  // elements (LDS instructions of one wave execute in order, so the reads
  // see this group's rows and the next group's writes follow them)
  auto pick_stage = [&](uint32_t (&rk)[KK][8]) {
    uint4* st = s_stage + wave * kStageU4;
#pragma unroll
    for (int u = 0; u < KK; ++u) st[lane + 64 * u] = stg[u];
    const uint16_t* sh = reinterpret_cast<const uint16_t*>(st);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) rk[kk][e] = sh[tof[kk][e]];
  };
  auto fetch_raw = [&](int grp, uint32_t (&rk)[KK][8], uint32_t (&rs)[KK][NS]) {
    int jl, q;
    code_pos(grp, jl, q);
    const uint16_t* xr = xbase + (int64_t)jl * xs3;
    const uint16_t* sg = sgb + (int64_t)jl * a.T;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int m = (16 * kk + 8 * hh) / C + e / CW;   // step of position 16kk + 8hh + e
        rk[kk][e] = xr[m * xs2 + raw_channel(kk, e, q)];
      }
#pragma unroll
      for (int l = 0; l < NS; ++l) rs[kk][l] = sg[(16 * kk + 8 * hh) / C + l];
    }
  };
  auto transform = [&](int grp, const uint32_t (&rk)[KK][8], const uint32_t (&rs)[KK][NS], bf16x8_t (&zh)[KK],
                       bf16x8_t (&zl)[KK], float& zz) {
    int jl, q;
    code_pos(grp, jl, q);
    zz = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      float rsg[NS];
#pragma unroll
      for (int l = 0; l < NS; ++l) {
        _Float16 sh;
        const uint16_t sb = (uint16_t)rs[kk][l];
        __builtin_memcpy(&sh, &sb, 2);
        rsg[l] = __builtin_amdgcn_rcpf((float)sh);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float wv = CPT <= 32 ? twt[kk][e] : wh[raw_channel(kk, e, q)];
        const float zf = (wv * bf16_to_f32(rk[kk][e])) * rsg[e / CW];
        const __bf16 z1 = (__bf16)zf;
        zz = fmaf(zf, zf, zz);
        zh[kk][e] = z1;
        zl[kk][e] = (__bf16)(zf - (float)z1);
      }
    }
  };

  // Lane constants of the norm product's B operand (zero in the second
  // half-wave).
  const uint32_t bn_lo = hh == 0 ? 0x3f803f80u : 0u;
  const uint32_t bn_hmask = hh == 0 ? 0xffff0000u : 0u;
  const uint32_t bn_one = hh == 0 ? 0x3f80u : 0u;

  // The next group's loads are issued before the current group is screened.
  // A wave with no group of its own (fewer than four groups in this
  // workgroup) still loads the last group, so every load is of a real row.
  constexpr int WS = kEncodeThreads / kWave;
  bf16x8_t bz[KK];
  uint32_t brk[TASQ ? KK : 1][8], brs[TASQ ? KK : 1][NS];
  const int grp_first = min(wave, ngroups - 1);   // ngroups >= 1: every workgroup has a token
  if constexpr (kStaged)
    fetch_stage(grp_first, brs);
  else if constexpr (TASQ)
    fetch_raw(grp_first, brk, brs);
  else
    fetch(grp_first, bz);
  for (int grp = wave; grp < ngroups; grp += WS) {
    bf16x8_t cz[KK], czlo[KK];
    float zz = 0.f;
    if constexpr (kStaged) {
      pick_stage(brk);
      uint32_t crs[KK][NS];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int l = 0; l < NS; ++l) crs[kk][l] = brs[kk][l];
      fetch_stage(min(grp + WS, ngroups - 1), brs);
      transform(grp, brk, crs, cz, czlo, zz);
    } else if constexpr (TASQ) {
      transform(grp, brk, brs, cz, czlo, zz);
      fetch_raw(min(grp + WS, ngroups - 1), brk, brs);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) cz[kk] = bz[kk];
      fetch(min(grp + WS, ngroups - 1), bz);
    }
    const int g = grp * 32 + n;
    const bool valid = CPT >= 32 || g < ncodes;

    if constexpr (!TASQ) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4 w = __builtin_bit_cast(uint4, cz[kk]);
        zz = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, w.x), zz, false);
        zz = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, w.y), zz, false);
        zz = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, w.z), zz, false);
        zz = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, w.w), zz, false);
      }
    }
    {
      // ||z||^2 of code n (both halves)
      const auto zs = __builtin_amdgcn_permlane32_swap(__float_as_uint(zz), __float_as_uint(zz), false, false);
      zz = __uint_as_float(zs[0]) + __uint_as_float(zs[1]);
    }
    // B operand of the norm product: [1, 1, 1, u] in the first half-wave,
    // zero in the second.  u >= ||z||^2 (1 + 2^-8) keeps the screened values
    // of every candidate that can come near the minimum positive, so their
    // bit patterns order like the values.
    // (bits + 0xffff) & 0xffff0000 rounds a positive float up to bf16.
    const uint32_t zzu = __float_as_uint(fmaf(zz, 1.f + 0x1p-8f, 1e-30f));
    const uint2 bnw = {bn_lo, ((zzu + 0xffffu) & bn_hmask) | bn_one};
    const s16x4_t bn = __builtin_bit_cast(s16x4_t, bnw);

    // Screening: every value is ||z - e_r||^2 + margin (fp32 MFMA); the key
    // replaces the low mantissa byte with the lane-local candidate number.
    // Keys are positive finite floats, so float min / median order them like
    // the screened values.  Two candidates per step: k1 = min3, and the new
    // second best is min(k2, median(k1_old, a, b)).
    float k1 = INFINITY, k2 = INFINITY;
    auto norms = [&](int t) {
      const f32x16_t z16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      return __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(an[t], bn, z16, 0, 0, 0);
    };
    auto screen = [&](f32x16_t acc, int t) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[t][kk], cz[kk], acc, 0, 0, 0);
        if constexpr (TASQ) {
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[t][kk], czlo[kk], acc, 0, 0, 0);
        }
      }
      return acc;
    };
    // Per candidate: the key of every screened value.
    auto select = [&](const f32x16_t& acc, int t) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        // low byte: the lane-local candidate number 16t + i
        const float ka = __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(acc[i]), (uint32_t)(16 * t + i), 0x07060500u));
        const float kb = __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(acc[i + 1]), (uint32_t)(16 * t + i + 1), 0x07060500u));
        const float md = __builtin_amdgcn_fmed3f(k1, ka, kb);
        k1 = fminf(k1, fminf(ka, kb));
        k2 = fminf(k2, md);
      }
    };
    // Per group of four: accumulators 4j .. 4j+3 of tile t are
    // the four consecutive codewords 32t + 8j + 4hh .. +3.  Only the smallest
    // screened value of a group gets a key (low byte: group number 4t + j);
    // the winning group is scored again below to find its member.
    auto select_groups = [&](const f32x16_t& acc, int t) {
      float gk[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float gm = fminf(fminf(acc[4 * j], acc[4 * j + 1]), fminf(acc[4 * j + 2], acc[4 * j + 3]));
        gk[j] = __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(gm), (uint32_t)(4 * t + j), 0x07060500u));
      }
#pragma unroll
      for (int j = 0; j < 4; j += 2) {
        const float md = __builtin_amdgcn_fmed3f(k1, gk[j], gk[j + 1]);
        k1 = fminf(k1, fminf(gk[j], gk[j + 1]));
        k2 = fminf(k2, md);
      }
    };
    // The norm product of tile t+1 is issued before tile t's selection.
    f32x16_t accn = norms(0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const f32x16_t acc = screen(accn, t);
      if (t + 1 < 8) accn = norms(t + 1);
      if constexpr (kGroups)
        select_groups(acc, t);
      else
        select(acc, t);
    }
    // Merge the two half-waves (lanes n and n+32 screen different codewords):
    // after the swaps both lanes of a code hold the first half's keys (a*)
    // and the second half's keys (b*) and take the same decision.
    const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(k1), __float_as_uint(k1), false, false);
    const auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(k2), __float_as_uint(k2), false, false);
    const uint32_t a1 = s1[0], b1 = s1[1], a2 = s2[0], b2 = s2[1];
    const float va1 = __uint_as_float(a1 & kmask), vb1 = __uint_as_float(b1 & kmask);
    const bool first = va1 <= vb1;
    const uint32_t wkey = first ? a1 : b1;
    const int whalf = first ? 0 : 1;
    const float t1 = first ? va1 : vb1;
    // second smallest screened value over both halves
    const float t2 = first ? fminf(__uint_as_float(a2 & kmask), vb1) : fminf(__uint_as_float(b2 & kmask), va1);
    // Exactness band.  A screened value carries at most kErr * (||e||^2 +
    // u) of fp32 rounding (the MFMA sums 4 + G exact bf16 products; |partial
    // sums| <= 2 (||e||^2 + u)).  Only candidates whose screened value can
    // reach the band matter; their distance is below Tb, so their norm is
    // below (||z|| + sqrt(Tb))^2 <= 2 (||z||^2 + Tb).  The key's low byte
    // adds < 2^-15 t1.
    // With Tb = 1.0625 t1 + ||z||^2 / 64 and nb = 2 (||z||^2 + Tb):
    //   eps = kErr (nb + 1.02 ||z||^2),
    //   thr = t1 (1 + 2^-14) + 2 eps  =  kA t1 + kB ||z||^2.
    // Pre-transformed keys: the MFMA sums 4 + 2G products (two split
    // terms), within 2 kErr; and the split sum differs from the exact
    // transformed value by < kSplit |z| (2^-16 from the split, ~2^-22 from
    // the fp32 product with the reciprocal of sigma), which moves a screened
    // value by < kSplit (||z||^2 + nb):
    //   eps = 2 kErr (nb + 1.02 ||z||^2) + kSplit (||z||^2 + nb).
    constexpr float kErr = (float)(2 * G + 16) * 0x1p-24f;
    constexpr float kSplit = 0x1.08p-16f;
    constexpr float kA = TASQ ? 1.f + 0x1p-14f + 8.5f * kErr + 4.25f * kSplit : 1.f + 0x1p-14f + 4.25f * kErr;
    constexpr float kB = TASQ ? 12.22f * kErr + 6.07f * kSplit : 6.11f * kErr;
    const float thr = fmaf(kA, t1, kB * zz);
    bool tie;
    int res;
    if constexpr (!kGroups) {
      tie = valid && !(t2 > thr);
      // candidate 16t + i of half-wave hh is codebook entry 32t + 8(i/4) + 4hh + i%4
      res = (int)(((wkey & 0x7cu) << 1) | (wkey & 3u)) | (whalf << 2);
    } else {
      // The winning group (codewords r0 .. r0+3) scored again in fp32: each
      // half-wave sums its eight positions per kk (the first half starting
      // from ||e||^2; pre-transformed keys add both split terms), the halves
      // are added.  At most G + 2 roundings (2G + 2 with two terms), each
      // within 2^-24 * 2 (||e||^2 + u), so these values obey the screened
      // values' error bound; they lack the margin u, so they are compared
      // with thr - u (one more rounding, within 2^-24 thr, inside the band's
      // 2^-15 t1 slack).  The candidate that gave t1 is re-scored to at most
      // thr - u, so the group's smallest value is always inside the band;
      // the code is exact unless another member (sv) or another group (t2)
      // also reaches it.
      const uint32_t gid = wkey & 0x1fu;
      const int r0 = (int)(32 * (gid >> 2) + 8 * (gid & 3u)) + 4 * whalf;
      const float thr_u = thr - __uint_as_float((zzu + 0xffffu) & 0xffff0000u);   // u as the norm product used it
      const float4 nf4 = *reinterpret_cast<const float4*>(&s_nf[r0]);
      const float nfv[4] = {nf4.x, nf4.y, nf4.z, nf4.w};
      float d[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float part = hh == 0 ? nfv[c] : 0.f;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const uint4 w = *reinterpret_cast<const uint4*>(&s_cb[cbrow(r0 + c) + 16 * kk + 8 * hh]);
          const uint4 z = __builtin_bit_cast(uint4, cz[kk]);
          part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, z.x), __builtin_bit_cast(bf16x2_t, w.x), part, false);
          part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, z.y), __builtin_bit_cast(bf16x2_t, w.y), part, false);
          part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, z.z), __builtin_bit_cast(bf16x2_t, w.z), part, false);
          part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, z.w), __builtin_bit_cast(bf16x2_t, w.w), part, false);
          if constexpr (TASQ) {
            const uint4 zl = __builtin_bit_cast(uint4, czlo[kk]);
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, zl.x), __builtin_bit_cast(bf16x2_t, w.x), part, false);
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, zl.y), __builtin_bit_cast(bf16x2_t, w.y), part, false);
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, zl.z), __builtin_bit_cast(bf16x2_t, w.z), part, false);
            part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, zl.w), __builtin_bit_cast(bf16x2_t, w.w), part, false);
          }
        }
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        d[c] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      }
      // smallest (lowest member on equal values) and the smallest of the rest
      float bv = d[0];
      int bc = 0;
#pragma unroll
      for (int c = 1; c < 4; ++c)
        if (d[c] < bv) {
          bv = d[c];
          bc = c;
        }
      float sv = INFINITY;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (c != bc) sv = fminf(sv, d[c]);
      tie = valid && !(t2 > thr && sv > thr_u);
      res = r0 + bc;
    }

    if (hh == 0) {
      if (tie)
        s_tq[atomicAdd(&s_tqn, 1)] = (uint16_t)g;
      else if (valid)
        ibase[g] = (uint8_t)res;
    }
  }

  // Codes inside the band: every codeword is scored exactly in fp64 (direct
  // form over the step-major positions) by the 64 lanes of a wave, four
  // candidates per lane; the smallest distance wins, then the lowest index.
  __syncthreads();
  const int nq = s_tqn;
  // exact fp64 scoring of queued code gq with joint vector zd (whole wave)
  auto score_code = [&](int gq, const double (&zd)[G]) {
    double best = INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int r = lane + 64 * c;
      if (r < a.K) {
        const uint4* cw = reinterpret_cast<const uint4*>(&s_cb[cbrow(r)]);
        double dist = 0.0;
#pragma unroll
        for (int c4 = 0; c4 < G / 8; ++c4) {
          const uint4 w = cw[c4];
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            // s_cb holds -2e, exactly
            const double d0 = zd[8 * c4 + 2 * k] + 0.5 * (double)bf16lo(ws[k]);
            const double d1 = zd[8 * c4 + 2 * k + 1] + 0.5 * (double)bf16hi(ws[k]);
            dist += d0 * d0;
            dist += d1 * d1;
          }
        }
        if (dist < best) {
          best = dist;
          bi = r;
        }
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const double ob = __shfl_xor(best, off);
      const int oi = __shfl_xor(bi, off);
      if (ob < best || (ob == best && oi < bi)) {
        best = ob;
        bi = oi;
      }
    }
    if (lane == 0) ibase[gq] = (uint8_t)bi;
  };
  if constexpr (!TASQ) {
    // raw bf16 words of a queued code (positions p = m*C + i: C contiguous
    // channels per step) as fp64
    auto load_zd = [&](int gq, double (&zd)[G]) {
      const int jl = gq >> LOG_CPT, q = gq & (CPT - 1);
      const uint16_t* xr = xbase + (int64_t)jl * xs3 + q * C;
      uint32_t zw[G / 2];
#pragma unroll
      for (int m = 0; m < TC; ++m) {
        const uint16_t* pm = xr + m * xs2;
        if constexpr (C >= 8) {
#pragma unroll
          for (int u = 0; u < C / 8; ++u) {
            const uint4 w = reinterpret_cast<const uint4*>(pm)[u];
            zw[m * C / 2 + 4 * u] = w.x;
            zw[m * C / 2 + 4 * u + 1] = w.y;
            zw[m * C / 2 + 4 * u + 2] = w.z;
            zw[m * C / 2 + 4 * u + 3] = w.w;
          }
        } else if constexpr (C == 4) {
          const uint2 w = *reinterpret_cast<const uint2*>(pm);
          zw[2 * m] = w.x;
          zw[2 * m + 1] = w.y;
        } else {
          zw[m] = *reinterpret_cast<const uint32_t*>(pm);
        }
      }
#pragma unroll
      for (int k = 0; k < G / 2; ++k) {
        zd[2 * k] = (double)bf16lo(zw[k]);
        zd[2 * k + 1] = (double)bf16hi(zw[k]);
      }
    };
    // exact fp64 distance of zd to codebook row r (s_cb holds -2e, exactly)
    auto exact_dist = [&](const double (&zd)[G], int r) {
      const uint4* cw = reinterpret_cast<const uint4*>(&s_cb[cbrow(r)]);
      double dist = 0.0;
#pragma unroll
      for (int c4 = 0; c4 < G / 8; ++c4) {
        const uint4 w = cw[c4];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const double d0 = zd[8 * c4 + 2 * k] + 0.5 * (double)bf16lo(ws[k]);
          const double d1 = zd[8 * c4 + 2 * k + 1] + 0.5 * (double)bf16hi(ws[k]);
          dist += d0 * d0;
          dist += d1 * d1;
        }
      }
      return dist;
    };
    // Batches of 32 queued codes per wave, screened again on the matrix cores
    // as in the loop above but keeping each half-wave's three best keys: the
    // band then holds at most its two best candidates, which are scored
    // exactly; a half with three or more inside the band sends its code to
    // the full scoring of every codeword.
    constexpr float kErrQ = (float)(2 * G + 16) * 0x1p-24f;
    constexpr float kAQ = 1.f + 0x1p-14f + 4.25f * kErrQ, kBQ = 6.11f * kErrQ;
    for (int bq = wave * 32; bq < nq; bq += WS * 32) {
      const bool qv = bq + n < nq;
      const int gq = s_tq[qv ? bq + n : bq];     // lanes past the end repeat a real code
      bf16x8_t qz[KK];
      {
        const int jl = gq >> LOG_CPT, q = gq & (CPT - 1);
        const uint16_t* xr = xbase + (int64_t)jl * xs3 + q * C;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const int p0 = 8 * (2 * kk + hh);
          const uint16_t* pz = xr + (int64_t)(p0 / C) * xs2 + (p0 % C);
          if constexpr (CW == 8) {
            qz[kk] = *reinterpret_cast<const bf16x8_t*>(pz);
          } else {
            uint32_t w[4];
#pragma unroll
            for (int l = 0; l < NL; ++l) {
              if constexpr (CW == 4) {
                const uint2 v = *reinterpret_cast<const uint2*>(pz + l * xs2);
                w[2 * l] = v.x;
                w[2 * l + 1] = v.y;
              } else {
                w[l] = *reinterpret_cast<const uint32_t*>(pz + l * xs2);
              }
            }
            qz[kk] = __builtin_bit_cast(bf16x8_t, (uint4){w[0], w[1], w[2], w[3]});
          }
        }
      }
      float zq = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint4 w = __builtin_bit_cast(uint4, qz[kk]);
        zq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.x), __builtin_bit_cast(bf16x2_t, w.x), zq, false);
        zq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.y), __builtin_bit_cast(bf16x2_t, w.y), zq, false);
        zq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.z), __builtin_bit_cast(bf16x2_t, w.z), zq, false);
        zq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w.w), __builtin_bit_cast(bf16x2_t, w.w), zq, false);
      }
      {
        const auto zs = __builtin_amdgcn_permlane32_swap(__float_as_uint(zq), __float_as_uint(zq), false, false);
        zq = __uint_as_float(zs[0]) + __uint_as_float(zs[1]);
      }
      const uint32_t zqu = __float_as_uint(fmaf(zq, 1.f + 0x1p-8f, 1e-30f));
      const uint2 bqw = {bn_lo, ((zqu + 0xffffu) & bn_hmask) | bn_one};
      const s16x4_t bnq = __builtin_bit_cast(s16x4_t, bqw);
      float k1 = INFINITY, k2 = INFINITY, k3 = INFINITY;
      // codeword operands from LDS (a runtime loop keeps the registers of this
      // rare phase below those of the screening loop)
#pragma unroll 1
      for (int t = 0; t < 8; ++t) {
        f32x16_t acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const s16x4_t rn = *reinterpret_cast<const s16x4_t*>(&s_nb[(32 * t + n) * 4]);
        acc = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(rn, bnq, acc, 0, 0, 0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8_t rv = *reinterpret_cast<const bf16x8_t*>(&s_cb[cbrow(32 * t + n) + 16 * kk + 8 * hh]);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rv, qz[kk], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float key = __uint_as_float(__builtin_amdgcn_perm(__float_as_uint(acc[i]), (uint32_t)(16 * t + i), 0x07060500u));
          const float n3 = __builtin_amdgcn_fmed3f(k2, k3, key);
          const float n2 = __builtin_amdgcn_fmed3f(k1, k2, key);
          k1 = fminf(k1, key);
          k2 = n2;
          k3 = n3;
        }
      }
      const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(k1), __float_as_uint(k1), false, false);
      const float t1 = fminf(__uint_as_float(s1[0] & kmask), __uint_as_float(s1[1] & kmask));
      const float thr = fmaf(kAQ, t1, kBQ * zq);
      const bool in1 = __uint_as_float(__float_as_uint(k1) & kmask) <= thr;
      const bool in2 = __uint_as_float(__float_as_uint(k2) & kmask) <= thr;
      const bool wide = __uint_as_float(__float_as_uint(k3) & kmask) <= thr;
      double zd[G];
      load_zd(gq, zd);
      double best = INFINITY;
      int bi = 0x7fffffff;
      // candidate number 16t + i of half hh is codebook row 32t + 8(i/4) + 4hh + i%4
      const uint32_t b1 = __float_as_uint(k1) & 0xffu, b2 = __float_as_uint(k2) & 0xffu;
      const int r1 = (int)(((b1 & 0x7cu) << 1) | (b1 & 3u)) | (hh << 2);
      const int r2 = (int)(((b2 & 0x7cu) << 1) | (b2 & 3u)) | (hh << 2);
      if (in1 && r1 < a.K) {
        best = exact_dist(zd, r1);
        bi = r1;
      }
      if (in2 && r2 < a.K) {
        const int r = r2;
        const double d = exact_dist(zd, r);
        if (d < best || (d == best && r < bi)) {
          best = d;
          bi = r;
        }
      }
      {
        const double ob = __shfl_xor(best, 32);
        const int oi = __shfl_xor(bi, 32);
        if (ob < best || (ob == best && oi < bi)) {
          best = ob;
          bi = oi;
        }
      }
      const bool full = wide || __shfl_xor((int)wide, 32) != 0;
      if (hh == 0 && qv && !full) ibase[gq] = (uint8_t)bi;
      uint64_t fm = __ballot(hh == 0 && qv && full);
      while (fm) {
        const int ln = __builtin_ctzll(fm);
        fm &= fm - 1;
        const int gf = __shfl(gq, ln);
        double zf[G];
        load_zd(gf, zf);
        score_code(gf, zf);
      }
    }
  } else {
    for (int e = wave; e < nq; e += WS) {
      const int gq = s_tq[e];
      const int jl = gq >> LOG_CPT, q = gq & (CPT - 1);
      const uint16_t* xr = xbase + (int64_t)jl * xs3;
      double zd[G];
#pragma unroll
      for (int p = 0; p < G; ++p) {
        const int m = p / C, d = q * C + (p % C);
        const int o = ph[d] & (D - 1);
        const double kv = (double)bf16_to_f32(xr[m * xs2 + o]);
        const double sg = f16_bits_to_f64(sgb[(int64_t)jl * a.T + m]);
        zd[p] = ((double)wh[o] * kv) / sg;
      }
      score_code(gq, zd);
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
