// LoopVQ fused decode attention for c = 4 channels per step per code (G = 16,
// 0.5 bit), T_c = 4, D = 128, no channel pre-transform: the headline
// geometry, laid out so that decoding an index costs one instruction.
//
// LoopVQ review (arXiv 2611.05304), section 3.4 step 3 (codebook on chip,
// lookup by index, RoPE after dequant from a precomputed table, Flash-
// Decoding split merge) and section 3.1 eq. (5) (step m reads coordinate
// i*T_c + m of the shared codeword).
//
// Layout choices for gfx950:
//   * Waves 0-1 serve steps 0-1 of the block, waves 2-3 steps 2-3.  The step
//     half is uniform in a wave, so the offset of a codeword's half in LDS
//     is an instruction immediate.
//   * A token is served by four lanes of a wave (16 tokens per wave).  Lane g
//     owns channels 16g .. 16g+15 and their RoPE partners 64+16g ..: chunks
//     4g .. 4g+3, which are the four bytes of dword g of the index row, and
//     chunks 16+4g .., the bytes of dword g+4.  A byte at a fixed position
//     turns into its LDS address with one v_mul_u32_u24 (SDWA byte select).
//   * Codewords sit in LDS as fp16, step-major halves of 16 bytes, with a
//     stride of three 16-byte slots.  The gathers are random, so they meet
//     bank conflicts whatever the stride (about 60% of the LDS-active time on
//     the 0.5-bit workload).  Both codebooks are rescaled by powers of two on
//     load (keys to fit fp16, values below 2^kHVLim), with the bf16 sinks and
//     recent rows counted in their ranges; the queries get a power-of-two
//     scale of their own.  The scales are folded back into scores and outputs.
//   * Rotation on packed fp16 pairs, scores as v_dot2_f32_f16 sums in fp32,
//     the four lanes of a token reduce with DPP inside a quad, online softmax
//     in base 2 whose running maximum may lag by kHLag, and P*V in packed
//     fp16 flushed into fp32 every kHFlush tokens.
// One workgroup serves one (batch, q-head, block, context split).
#include "common.h"
#include "kernels.h"

namespace loopvq {

namespace {

typedef _Float16 hh2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ hh2_t as_hh2(uint32_t w) { return __builtin_bit_cast(hh2_t, w); }

__device__ __forceinline__ uint32_t pack_hh2(float a, float b) {
  const _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// fp16 partial sums of P*V: weights <= 2^kHLag, |v| <= 2^kHVLim, kHFlush tokens
// per lane between flushes keep a partial below 2^(3+7+4) = 16384.
constexpr int kHFlush = 16, kHLag = 3, kHVLim = 7;
constexpr int kCWS = 3;                 // LDS slots of 16 bytes per codeword (2 used)

// LDS byte address of codeword `byte k of w`: k * 48 in one SDWA multiply.
template <int K>
__device__ __forceinline__ uint32_t cw_addr(uint32_t w) {
  return __umul24(__builtin_amdgcn_ubfe(w, 8 * K, 8), 16 * kCWS);
}

}  // namespace

template <int HS>
__device__ __forceinline__ void decode_half_body(const DecodeArgs& a, const uint4* s_k, const uint4* s_v,
                                                 float (*s_red)[2][130], int b, int hq, int h, int beta, int split,
                                                 int shk, int shv, int shq) {
  constexpr int D = 128, HD = 64, TC = 4, C = 4, CPT = D / C;
  constexpr int NW = kDecodeThreads / kWave, SPW = 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wt = wave & 1;              // which 16 tokens of an iteration
  const int slot = lane >> 2, g = lane & 3;
  const char* kbase = reinterpret_cast<const char*>(s_k) + 16 * HS;
  const char* vbase = reinterpret_cast<const char*>(s_v) + 16 * HS;

  // queries: steps 2HS + ml; chunk pair k (chunk 4g + k and its partner), channel pair ip
  const int t_lo = max(a.step0, beta * TC), t_hi = min(a.step0 + a.n_steps, (beta + 1) * TC);
  uint32_t qv[2][4][2][2];
  const float qsc = ldexpf(1.f, -shq);
#pragma unroll
  for (int ml = 0; ml < 2; ++ml) {
    const int t = beta * TC + 2 * HS + ml;
    const bool act = t >= t_lo && t < t_hi;
    const uint16_t* qr = a.q + (((int64_t)b * a.Hq + hq) * a.n_steps + (act ? t - a.step0 : 0)) * D;
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int ip = 0; ip < 2; ++ip) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(qr + p * HD + 16 * g + 4 * k + 2 * ip);
          qv[ml][k][p][ip] = act ? pack_hh2(bf16lo(w) * qsc, bf16hi(w) * qsc) : 0u;
        }
  }
  const float sscale = a.qscale * ldexpf(1.f, shk + shq);

  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};
  float acc[2][4][2][4];
  uint32_t acc16[2][4][2][2];
#pragma unroll
  for (int ml = 0; ml < 2; ++ml)
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[ml][k][p][c] = 0.f;
        acc16[ml][k][p][0] = acc16[ml][k][p][1] = 0u;
      }

  int nb = a.N;
  if (a.seq_len) nb = max(0, min(a.seq_len[b], a.N));
  const int tok_lo = split * a.tok_per_split;
  const int tok_hi = min(nb, tok_lo + a.tok_per_split);
  const int n_sink = split == 0 ? a.n_s : 0;
  const int n_bf = n_sink + (split == 0 ? a.n_r : 0);
  const int64_t irow0 = (((int64_t)b * a.H + h) * a.n_blk + beta) * (int64_t)a.N_cap;
  const int64_t sink0 = (((int64_t)b * a.H + h) * a.T + beta * TC) * (int64_t)a.n_s;
  const int64_t rec0 = (((int64_t)b * a.H + h) * a.T + beta * TC) * (int64_t)a.r_cap;
  const uint16_t* rope16 = reinterpret_cast<const uint16_t*>(a.rope);
  const float ksc = ldexpf(1.f, -shk), vsc = ldexpf(1.f, -shv);

  // Kw[c]: half of chunk 4g + c (c < 4) or of its partner 16 + 4g + (c - 4);
  // words [ml][ip].  CS[k]: sin/cos quad of chunk 4g + k.
  auto scores = [&](const uint32_t (&Kw)[8][4], const uint4 (&CS)[4], float (&sc)[2]) {
    sc[0] = sc[1] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int ml = 0; ml < 2; ++ml) {
#pragma unroll
        for (int ip = 0; ip < 2; ++ip) {
          const uint4 q4 = CS[k];
          const hh2_t c2 = as_hh2(ip ? q4.y : q4.x), s2 = as_hh2(ip ? q4.w : q4.z);
          const hh2_t x1 = as_hh2(Kw[k][2 * ml + ip]), x2 = as_hh2(Kw[k + 4][2 * ml + ip]);
          const hh2_t r1 = x1 * c2 - x2 * s2;
          const hh2_t r2 = x2 * c2 + x1 * s2;
          sc[ml] = __builtin_amdgcn_fdot2(r1, as_hh2(qv[ml][k][0][ip]), sc[ml], false);
          sc[ml] = __builtin_amdgcn_fdot2(r2, as_hh2(qv[ml][k][1][ip]), sc[ml], false);
        }
      }
    }
#pragma unroll
    for (int ml = 0; ml < 2; ++ml) sc[ml] = group_sum<4>(sc[ml]) * sscale;
  };
  auto flush = [&]() {
#pragma unroll
    for (int ml = 0; ml < 2; ++ml)
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int ip = 0; ip < 2; ++ip) {
            add_f16x2(acc16[ml][k][p][ip], acc[ml][k][p][2 * ip], acc[ml][k][p][2 * ip + 1]);
            acc16[ml][k][p][ip] = 0u;
          }
  };
  auto accumulate = [&](const float (&sc)[2], const uint32_t (&Vw)[8][4], bool valid) {
    if (!valid) return;
#pragma unroll
    for (int ml = 0; ml < 2; ++ml) {
      const float s = sc[ml];
      if (s > mrow[ml] + (float)kHLag) {
        const float alpha = __builtin_amdgcn_exp2f(mrow[ml] - s);
        const hh2_t a2 = {(_Float16)alpha, (_Float16)alpha};
        lrow[ml] *= alpha;
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[ml][k][p][c] *= alpha;
#pragma unroll
            for (int ip = 0; ip < 2; ++ip)
              acc16[ml][k][p][ip] = __builtin_bit_cast(uint32_t, as_hh2(acc16[ml][k][p][ip]) * a2);
          }
        mrow[ml] = s;
      }
      const float pr = __builtin_amdgcn_exp2f(s - mrow[ml]);
      lrow[ml] += pr;
      const hh2_t p2 = {(_Float16)pr, (_Float16)pr};
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int ip = 0; ip < 2; ++ip) {
            const hh2_t v2 = as_hh2(Vw[k + 4 * p][2 * ml + ip]);
            acc16[ml][k][p][ip] = __builtin_bit_cast(uint32_t, v2 * p2 + as_hh2(acc16[ml][k][p][ip]));
          }
    }
  };
  auto load_cs = [&](int pos, uint4 (&CS)[4]) {
    const uint4* row = reinterpret_cast<const uint4*>(rope16 + (int64_t)pos * D);
#pragma unroll
    for (int k = 0; k < 4; ++k) CS[k] = row[4 * g + k];
  };
  auto gather = [&](const char* base, uint32_t addr, uint32_t (&out)[4]) {
    const uint4 x = *reinterpret_cast<const uint4*>(base + addr);
    out[0] = x.x;
    out[1] = x.y;
    out[2] = x.z;
    out[3] = x.w;
  };

  // Sinks and the recent window (split 0 only), straight from the bf16 rows,
  // scaled like the codebooks.  Sink s sits at position s, recent token r at
  // n_s + N_b + r.
  for (int base = 0; base < n_bf; base += 2 * SPW) {
    const int item = base + wt * SPW + slot;
    const bool valid = item < n_bf;
    const int it = valid ? item : 0;
    const bool is_rec = it >= n_sink;
    const int pos = is_rec ? a.n_s + nb + (it - n_sink) : it;
    uint32_t Kw[8][4], Vw[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int d0 = (c >> 2) * HD + 16 * g + 4 * (c & 3);
#pragma unroll
      for (int ml = 0; ml < 2; ++ml) {
        const int m = 2 * HS + ml;
        const uint16_t* kr = (is_rec ? a.rk + (rec0 + (int64_t)m * a.r_cap + (it - n_sink)) * D
                                     : a.sk + (sink0 + (int64_t)m * a.n_s + it) * D) + d0;
        const uint16_t* vr = (is_rec ? a.rv + (rec0 + (int64_t)m * a.r_cap + (it - n_sink)) * D
                                     : a.sv + (sink0 + (int64_t)m * a.n_s + it) * D) + d0;
#pragma unroll
        for (int ip = 0; ip < 2; ++ip) {
          const uint32_t x = *reinterpret_cast<const uint32_t*>(kr + 2 * ip);
          const uint32_t y = *reinterpret_cast<const uint32_t*>(vr + 2 * ip);
          Kw[c][2 * ml + ip] = pack_hh2(bf16lo(x) * ksc, bf16hi(x) * ksc);
          Vw[c][2 * ml + ip] = pack_hh2(bf16lo(y) * vsc, bf16hi(y) * vsc);
        }
      }
    }
    uint4 CS[4];
    load_cs(pos, CS);
    float sc[2];
    scores(Kw, CS, sc);
    accumulate(sc, Vw, valid);
    flush();
  }

  // Context tokens: index dwords g and g + 4 of the K and V rows, loaded one
  // iteration ahead with the sin/cos quads.
  const int n_tok = max(0, tok_hi - tok_lo);
  const int my = wt * SPW + slot;
  uint32_t kd[2], vd[2];
  uint4 CS[4];
  auto load_rows = [&](int base, int& jj) {
    const int it = base + my;
    jj = tok_lo + (it < n_tok ? it : n_tok - 1);   // always a real row
    const uint32_t* kr = reinterpret_cast<const uint32_t*>(a.kidx + (irow0 + jj) * CPT);
    const uint32_t* vr = reinterpret_cast<const uint32_t*>(a.vidx + (irow0 + jj) * CPT);
    kd[0] = kr[g];
    kd[1] = kr[g + 4];
    vd[0] = vr[g];
    vd[1] = vr[g + 4];
  };
  if (n_tok > 0) {
    int jj;
    load_rows(0, jj);
    load_cs(a.n_s + jj, CS);
  }
  int since_flush = 0;
  for (int base = 0; base < n_tok; base += 2 * SPW) {
    const bool valid = base + my < n_tok;
    uint32_t ka[8], va[8];
    ka[0] = cw_addr<0>(kd[0]); ka[1] = cw_addr<1>(kd[0]); ka[2] = cw_addr<2>(kd[0]); ka[3] = cw_addr<3>(kd[0]);
    ka[4] = cw_addr<0>(kd[1]); ka[5] = cw_addr<1>(kd[1]); ka[6] = cw_addr<2>(kd[1]); ka[7] = cw_addr<3>(kd[1]);
    va[0] = cw_addr<0>(vd[0]); va[1] = cw_addr<1>(vd[0]); va[2] = cw_addr<2>(vd[0]); va[3] = cw_addr<3>(vd[0]);
    va[4] = cw_addr<0>(vd[1]); va[5] = cw_addr<1>(vd[1]); va[6] = cw_addr<2>(vd[1]); va[7] = cw_addr<3>(vd[1]);
    int jn;
    load_rows(base + 2 * SPW, jn);
    uint32_t Kw[8][4], Vw[8][4];
#pragma unroll
    for (int c = 0; c < 8; ++c) gather(kbase, ka[c], Kw[c]);
#pragma unroll
    for (int c = 0; c < 8; ++c) gather(vbase, va[c], Vw[c]);
    float sc[2];
    scores(Kw, CS, sc);
    load_cs(a.n_s + jn, CS);
    accumulate(sc, Vw, valid);
    if (++since_flush == kHFlush) {
      flush();
      since_flush = 0;
    }
  }
  flush();

  // merge the 16 token slots of the wave (lanes with equal g)
#pragma unroll
  for (int off = 4; off < kWave; off <<= 1) {
#pragma unroll
    for (int ml = 0; ml < 2; ++ml) {
      const float om = __shfl_xor(mrow[ml], off);
      const float ol = __shfl_xor(lrow[ml], off);
      const float mm = fmaxf(mrow[ml], om);
      const float a1 = mrow[ml] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrow[ml] - mm);
      const float a2 = om == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(om - mm);
      lrow[ml] = lrow[ml] * a1 + ol * a2;
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float oa = __shfl_xor(acc[ml][k][p][c], off);
            acc[ml][k][p][c] = acc[ml][k][p][c] * a1 + oa * a2;
          }
      mrow[ml] = mm;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int ml = 0; ml < 2; ++ml) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int c = 0; c < 4; ++c) s_red[wave][ml][p * HD + 16 * g + 4 * k + c] = acc[ml][k][p][c];
      if (g == 0) {
        s_red[wave][ml][D] = mrow[ml];
        s_red[wave][ml][D + 1] = lrow[ml];
      }
    }
  }
  (void)NW;
}

__global__ __launch_bounds__(kDecodeThreads) void decode_half_kernel(DecodeArgs a) {
  constexpr int D = 128, TC = 4, G = 16, NW = kDecodeThreads / kWave;
  __shared__ __attribute__((aligned(16))) uint4 s_k[256 * kCWS];
  __shared__ __attribute__((aligned(16))) uint4 s_v[256 * kCWS];
  __shared__ float s_red[NW][2][D + 2];
  __shared__ float s_amax[3][NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x;
  const int hq = blockIdx.y;
  const int h = hq / a.gqa;
  const int b = blockIdx.z / a.n_blk_serv;
  const int beta = a.blk0 + (blockIdx.z - b * a.n_blk_serv);
  const int t_lo = max(a.step0, beta * TC), t_hi = min(a.step0 + a.n_steps, (beta + 1) * TC);

  // ---- codebooks -> LDS (fp16, step-major halves), power-of-two range scaling
  const int64_t cbo = ((int64_t)h * a.n_blk + beta) * a.K * G;
  const int r = tid;   // one row per thread
  float kx[G], vx[G];
  float mq, mk, mv;   // the bf16 sinks and recent rows share the codebooks' scales
  decode_input_absmax(a, b, hq, 1, h, t_lo, t_hi, split == 0, nullptr, mq, mk, mv);
  if (r < a.K) {
    const uint4* pk = reinterpret_cast<const uint4*>(a.kcb + cbo + r * G);
    const uint4* pv = reinterpret_cast<const uint4*>(a.vcb + cbo + r * G);
#pragma unroll
    for (int c4 = 0; c4 < G / 8; ++c4) {
      const uint4 x = pk[c4], y = pv[c4];
      const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        kx[8 * c4 + 2 * w] = bf16lo(xw[w]);
        kx[8 * c4 + 2 * w + 1] = bf16hi(xw[w]);
        vx[8 * c4 + 2 * w] = bf16lo(yw[w]);
        vx[8 * c4 + 2 * w + 1] = bf16hi(yw[w]);
      }
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      mk = fmaxf(mk, fabsf(kx[u]));
      mv = fmaxf(mv, fabsf(vx[u]));
    }
  } else {
#pragma unroll
    for (int u = 0; u < G; ++u) kx[u] = vx[u] = 0.f;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    mq = fmaxf(mq, __shfl_xor(mq, off));
    mk = fmaxf(mk, __shfl_xor(mk, off));
    mv = fmaxf(mv, __shfl_xor(mv, off));
  }
  if (lane == 0) {
    s_amax[0][wave] = mk;
    s_amax[1][wave] = mv;
    s_amax[2][wave] = mq;
  }
  __syncthreads();
  mk = fmaxf(fmaxf(s_amax[0][0], s_amax[0][1]), fmaxf(s_amax[0][2], s_amax[0][3]));
  mv = fmaxf(fmaxf(s_amax[1][0], s_amax[1][1]), fmaxf(s_amax[1][2], s_amax[1][3]));
  mq = fmaxf(fmaxf(s_amax[2][0], s_amax[2][1]), fmaxf(s_amax[2][2], s_amax[2][3]));
  const int shk = pow2_range_shift(mk, 14), shv = pow2_range_shift(mv, kHVLim), shq = pow2_range_shift(mq, 14);
  {
    const float sk = ldexpf(1.f, -shk), sv = ldexpf(1.f, -shv);
    uint32_t kw[8], vw[8];   // [m][pair]: step m, channels (2*pair, 2*pair+1)
#pragma unroll
    for (int m = 0; m < TC; ++m)
#pragma unroll
      for (int ip = 0; ip < 2; ++ip) {
        // joint coordinate of channel i at step m is i*T_c + m
        kw[2 * m + ip] = pack_hh2(kx[(2 * ip) * TC + m] * sk, kx[(2 * ip + 1) * TC + m] * sk);
        vw[2 * m + ip] = pack_hh2(vx[(2 * ip) * TC + m] * sv, vx[(2 * ip + 1) * TC + m] * sv);
      }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s_k[r * kCWS + u] = make_uint4(kw[4 * u], kw[4 * u + 1], kw[4 * u + 2], kw[4 * u + 3]);
      s_v[r * kCWS + u] = make_uint4(vw[4 * u], vw[4 * u + 1], vw[4 * u + 2], vw[4 * u + 3]);
    }
  }
  __syncthreads();

  if (wave >> 1)
    decode_half_body<1>(a, s_k, s_v, s_red, b, hq, h, beta, split, shk, shv, shq);
  else
    decode_half_body<0>(a, s_k, s_v, s_red, b, hq, h, beta, split, shk, shv, shq);
  __syncthreads();

  // ---- merge the two waves of each step half
  const float osc = ldexpf(1.f, shv);
  for (int x = tid; x < TC * D; x += kDecodeThreads) {
    const int m = x / D, d = x - m * D;
    const int t = beta * TC + m;
    if (t < t_lo || t >= t_hi) continue;
    const int w0 = 2 * (m >> 1), ml = m & 1;
    const float m0 = s_red[w0][ml][D], m1 = s_red[w0 + 1][ml][D];
    const float mm = fmaxf(m0, m1);
    float num = 0.f, den = 0.f;
    if (mm != -INFINITY) {
      const float f0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - mm);
      const float f1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mm);
      num = f0 * s_red[w0][ml][d] + f1 * s_red[w0 + 1][ml][d];
      den = f0 * s_red[w0][ml][D + 1] + f1 * s_red[w0 + 1][ml][D + 1];
    }
    const int64_t row = ((int64_t)b * a.Hq + hq) * a.n_steps + (t - a.step0);
    const float o = den > 0.f ? num / den * osc : 0.f;
    const float l = den > 0.f ? (mm + __log2f(den)) * 0.69314718055994531f : -INFINITY;
    if (a.out) {
      // one split: the rows go straight to out / lse (the merge of a single
      // partial returns it unchanged)
      a.out[row * D + d] = o;
      if (d == 0 && a.lse) a.lse[row] = l;
    } else {
      float* dst = a.ws + (row * a.n_split + split) * (D + 1);
      dst[d] = o;
      if (d == 0) dst[D] = l;
    }
  }
}

hipError_t launch_decode_half(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.Hq, a.B * a.n_blk_serv);
  hipLaunchKernelGGL(decode_half_kernel, grid, dim3(kDecodeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace loopvq
