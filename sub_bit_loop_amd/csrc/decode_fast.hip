// LoopVQ fused decode attention, specialised for blocks of T_c = 4 loop steps
// with c = 8 (G = 32, 0.25 bit) channels per step per code, D = 128, no
// channel pre-transform (c = 4 has its own layout in decode_half.hip; the
// kernel template below still covers it), and the single-step variant.
//
// LoopVQ review (arXiv 2611.05304), section 3.4 step 3 (codebook on chip,
// lookup by index, RoPE from a precomputed table after dequant, Flash-
// Decoding split merge) and section 3.1 eq. (5) (step m reads coordinate
// i*T_c + m of the shared codeword).
//
// Layout choices for gfx950:
//   * Both codebooks sit in LDS as fp16, step-major inside a codeword (word
//     (m, channel pair) at m*2c + 4*pair bytes).  The first half of a codeword
//     holds steps 0-1, the second steps 2-3; a lane reads the half of its two
//     steps with c/4 ds_read_b128.
//   * A token is served by 8 lanes: lane (h, g) takes steps {2h, 2h+1} and the
//     chunk pairs (q, q + D/(2c)) for q = g, g+4, ..., i.e. exactly the
//     channel pairs that RoPE rotates together.  Every index byte is decoded
//     once for all four steps.
//   * Rotation runs on packed fp16 pairs of adjacent channels, scores are
//     v_dot2_f32_f16 sums in fp32, the four same-step lanes reduce with DPP
//     inside a quad, the softmax is online (base 2) and P*V accumulates packed
//     fp16 pairs that are flushed into fp32 every kFlush tokens.
//   * Codebooks are rescaled by a power of two on load so that keys fit fp16
//     and values stay below 2^kVLim (the bf16 sinks and recent rows count in
//     those ranges), and the queries by one of their own; the scales are
//     folded back into scores and outputs.
// One workgroup serves one (batch, q-head, block, context split); q-heads of a
// GQA group gather the same rows in separate workgroups.
#include "common.h"
#include "kernels.h"

namespace loopvq {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2_t as_h2(uint32_t w) { return __builtin_bit_cast(h2_t, w); }

// Power-of-two exponent s >= 0 with max_abs * 2^-s <= 2^lim.
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  const _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// P*V accumulates in packed fp16 for kFlush tokens per lane and is then added
// into fp32.  With the running max allowed to lag by at most kLag (weights
// <= 2^kLag) and |v| <= 2^kVLim, a partial sum stays below 2^(3+7+4) = 16384.
constexpr int kFlush = 16, kLag = 3, kVLim = 7;

template <int C>
__global__ __launch_bounds__(kDecodeThreads) void decode_fast_kernel(DecodeArgs a) {
  constexpr int D = 128, HD = 64, TC = 4, G = C * TC, CPT = D / C;
  constexpr int NP = HD / C;          // RoPE chunk pairs per token (16 or 8)
  constexpr int NPL = NP / 4;         // chunk pairs per lane (4 or 2)
  constexpr int NCW = 2 * NPL;        // codewords gathered per lane per token
  constexpr int QW = C / 4;           // uint4 per codeword half (two steps)
  constexpr int DW = C / 2;           // dwords per step of a codeword
  constexpr int RW = CPT / 16;        // uint4 per index row
  constexpr int LPT = 8, SPW = kWave / LPT, NW = kDecodeThreads / kWave;
  __shared__ __attribute__((aligned(16))) uint4 s_k[256 * 2 * QW];
  __shared__ __attribute__((aligned(16))) uint4 s_v[256 * 2 * QW];
  __shared__ float s_red[NW][TC][D + 2];
  __shared__ float s_amax[3][NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sl = lane & 7, slot = lane >> 3;
  const int hs = sl >> 2, g = sl & 3;           // step half, chunk group
  const int split = blockIdx.x;
  const int hq = blockIdx.y;
  const int h = hq / a.gqa;
  const int b = blockIdx.z / a.n_blk_serv;
  const int beta = a.blk0 + (blockIdx.z - b * a.n_blk_serv);
  const int t_lo = max(a.step0, beta * TC), t_hi = min(a.step0 + a.n_steps, (beta + 1) * TC);

  // ---- codebooks -> LDS (fp16, step-major), with power-of-two range scaling
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
  const int shk = pow2_range_shift(mk, 14), shv = pow2_range_shift(mv, kVLim), shq = pow2_range_shift(mq, 14);
  const float qsc = ldexpf(1.f, -shq);
  {
    const float sk = ldexpf(1.f, -shk), sv = ldexpf(1.f, -shv);
    uint32_t kw[2 * C], vw[2 * C];   // [m][pair]: step m, channels (2*pair, 2*pair+1)
#pragma unroll
    for (int m = 0; m < TC; ++m) {
#pragma unroll
      for (int ip = 0; ip < DW; ++ip) {
        // joint coordinate of channel i at step m is i*T_c + m
        kw[m * DW + ip] = pack_h2(kx[(2 * ip) * TC + m] * sk, kx[(2 * ip + 1) * TC + m] * sk);
        vw[m * DW + ip] = pack_h2(vx[(2 * ip) * TC + m] * sv, vx[(2 * ip + 1) * TC + m] * sv);
      }
    }
#pragma unroll
    for (int u = 0; u < 2 * QW; ++u) {
      s_k[r * 2 * QW + u] = make_uint4(kw[4 * u], kw[4 * u + 1], kw[4 * u + 2], kw[4 * u + 3]);
      s_v[r * 2 * QW + u] = make_uint4(vw[4 * u], vw[4 * u + 1], vw[4 * u + 2], vw[4 * u + 3]);
    }
  }

  // ---- queries of this lane: steps 2hs+ml, chunk pairs k, partner p, channel pair ip
  uint32_t qv[2][NPL][2][DW];
#pragma unroll
  for (int ml = 0; ml < 2; ++ml) {
    const int t = beta * TC + 2 * hs + ml;
    const bool act = t >= t_lo && t < t_hi;
    const uint16_t* qr = a.q + (((int64_t)b * a.Hq + hq) * a.n_steps + (act ? t - a.step0 : 0)) * D;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int d0 = p * HD + C * (g + 4 * k);
#pragma unroll
        for (int ip = 0; ip < DW; ++ip) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(qr + d0 + 2 * ip);
          qv[ml][k][p][ip] = act ? pack_h2(bf16lo(w) * qsc, bf16hi(w) * qsc) : 0u;
        }
      }
    }
  }
  const float sscale = a.qscale * ldexpf(1.f, shk + shq);

  float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};
  float acc[2][NPL][2][C];
  uint32_t acc16[2][NPL][2][DW];
#pragma unroll
  for (int ml = 0; ml < 2; ++ml)
#pragma unroll
    for (int k = 0; k < NPL; ++k)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int c = 0; c < C; ++c) acc[ml][k][p][c] = 0.f;
#pragma unroll
        for (int ip = 0; ip < DW; ++ip) acc16[ml][k][p][ip] = 0u;
      }
  __syncthreads();

  int nb = a.N;
  if (a.seq_len) nb = max(0, min(a.seq_len[b], a.N));
  const int tok_lo = split * a.tok_per_split;
  const int tok_hi = min(nb, tok_lo + a.tok_per_split);
  // bf16 items (sinks, then the recent window) are served by split 0.
  const int n_sink = split == 0 ? a.n_s : 0;
  const int n_bf = n_sink + (split == 0 ? a.n_r : 0);
  const int64_t irow0 = (((int64_t)b * a.H + h) * a.n_blk + beta) * (int64_t)a.N_cap;
  const int64_t sink0 = (((int64_t)b * a.H + h) * a.T + beta * TC) * (int64_t)a.n_s;
  const int64_t rec0 = (((int64_t)b * a.H + h) * a.T + beta * TC) * (int64_t)a.r_cap;
  const uint16_t* rope16 = reinterpret_cast<const uint16_t*>(a.rope);
  const float ksc = ldexpf(1.f, -shk), vsc = ldexpf(1.f, -shv);

  // Codeword halves of one token: Kw[c] for c < NPL are chunks g + 4c, the
  // rest their RoPE partners; each half is C dwords (two steps x DW words).
  // CS[k][u]: sin/cos quads of chunk g + 4k (quad u covers 4 frequencies).
  auto scores = [&](const uint32_t (&Kw)[NCW][C], const uint4 (&CS)[NPL][QW], float (&sc)[2]) {
    sc[0] = sc[1] = 0.f;
#pragma unroll
    for (int k = 0; k < NPL; ++k) {
#pragma unroll
      for (int ml = 0; ml < 2; ++ml) {
#pragma unroll
        for (int ip = 0; ip < DW; ++ip) {
          const uint4 q4 = CS[k][ip >> 1];
          const h2_t c2 = as_h2((ip & 1) ? q4.y : q4.x), s2 = as_h2((ip & 1) ? q4.w : q4.z);
          const h2_t x1 = as_h2(Kw[k][ml * DW + ip]), x2 = as_h2(Kw[k + NPL][ml * DW + ip]);
          const h2_t r1 = x1 * c2 - x2 * s2;
          const h2_t r2 = x2 * c2 + x1 * s2;
          sc[ml] = __builtin_amdgcn_fdot2(r1, as_h2(qv[ml][k][0][ip]), sc[ml], false);
          sc[ml] = __builtin_amdgcn_fdot2(r2, as_h2(qv[ml][k][1][ip]), sc[ml], false);
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
      for (int k = 0; k < NPL; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int ip = 0; ip < DW; ++ip) {
            add_f16x2(acc16[ml][k][p][ip], acc[ml][k][p][2 * ip], acc[ml][k][p][2 * ip + 1]);
            acc16[ml][k][p][ip] = 0u;
          }
  };
  // Online softmax (base 2) and P*V.  The running maximum moves only when a
  // score exceeds it by more than kLag, which keeps rescaling rare.
  auto accumulate = [&](const float (&sc)[2], const uint32_t (&Vw)[NCW][C], bool valid) {
    if (!valid) return;
#pragma unroll
    for (int ml = 0; ml < 2; ++ml) {
      const float s = sc[ml];
      if (s > mrow[ml] + (float)kLag) {
        const float alpha = __builtin_amdgcn_exp2f(mrow[ml] - s);
        const h2_t a2 = {(_Float16)alpha, (_Float16)alpha};
        lrow[ml] *= alpha;
#pragma unroll
        for (int k = 0; k < NPL; ++k)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
#pragma unroll
            for (int c = 0; c < C; ++c) acc[ml][k][p][c] *= alpha;
#pragma unroll
            for (int ip = 0; ip < DW; ++ip)
              acc16[ml][k][p][ip] = __builtin_bit_cast(uint32_t, as_h2(acc16[ml][k][p][ip]) * a2);
          }
        mrow[ml] = s;
      }
      const float pr = __builtin_amdgcn_exp2f(s - mrow[ml]);
      lrow[ml] += pr;
      const h2_t p2 = {(_Float16)pr, (_Float16)pr};
#pragma unroll
      for (int k = 0; k < NPL; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int ip = 0; ip < DW; ++ip) {
            const h2_t v2 = as_h2(Vw[k + NPL * p][ml * DW + ip]);
            acc16[ml][k][p][ip] = __builtin_bit_cast(uint32_t, v2 * p2 + as_h2(acc16[ml][k][p][ip]));
          }
    }
  };
  auto load_cs = [&](int pos, uint4 (&CS)[NPL][QW]) {
    const uint4* row = reinterpret_cast<const uint4*>(rope16 + (int64_t)pos * D);
#pragma unroll
    for (int k = 0; k < NPL; ++k)
#pragma unroll
      for (int u = 0; u < QW; ++u) CS[k][u] = row[(C / 4) * (g + 4 * k) + u];
  };
  auto gather = [&](const uint4* tab, uint32_t cw, uint32_t (&out)[C]) {
#pragma unroll
    for (int u = 0; u < QW; ++u) {
      const uint4 x = tab[(2 * cw + hs) * QW + u];
      out[4 * u] = x.x;
      out[4 * u + 1] = x.y;
      out[4 * u + 2] = x.z;
      out[4 * u + 3] = x.w;
    }
  };

  // Sinks and the recent window (split 0 only): straight from the bf16 rows,
  // scaled like the codebooks.  Sink s sits at position s, recent token r at
  // n_s + N_b + r.
  for (int base = 0; base < n_bf; base += NW * SPW) {
    const int item = base + wave * SPW + slot;
    const bool valid = item < n_bf;
    const int it = valid ? item : 0;
    const bool is_rec = it >= n_sink;
    const int pos = is_rec ? a.n_s + nb + (it - n_sink) : it;
    uint32_t Kw[NCW][C], Vw[NCW][C];
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      const int k = c % NPL, p = c / NPL;
      const int d0 = p * HD + C * (g + 4 * k);
#pragma unroll
      for (int ml = 0; ml < 2; ++ml) {
        const int m = 2 * hs + ml;
        const uint16_t* kr = (is_rec ? a.rk + (rec0 + (int64_t)m * a.r_cap + (it - n_sink)) * D
                                     : a.sk + (sink0 + (int64_t)m * a.n_s + it) * D) + d0;
        const uint16_t* vr = (is_rec ? a.rv + (rec0 + (int64_t)m * a.r_cap + (it - n_sink)) * D
                                     : a.sv + (sink0 + (int64_t)m * a.n_s + it) * D) + d0;
#pragma unroll
        for (int ip = 0; ip < DW; ++ip) {
          const uint32_t x = *reinterpret_cast<const uint32_t*>(kr + 2 * ip);
          const uint32_t y = *reinterpret_cast<const uint32_t*>(vr + 2 * ip);
          Kw[c][ml * DW + ip] = pack_h2(bf16lo(x) * ksc, bf16hi(x) * ksc);
          Vw[c][ml * DW + ip] = pack_h2(bf16lo(y) * vsc, bf16hi(y) * vsc);
        }
      }
    }
    uint4 CS[NPL][QW];
    load_cs(pos, CS);
    float sc[2];
    scores(Kw, CS, sc);
    accumulate(sc, Vw, valid);
    flush();
  }

  // Context tokens.  The index rows and the sin/cos quads of the next
  // iteration are loaded as soon as the current ones are consumed.
  const int n_tok = max(0, tok_hi - tok_lo);
  const int my = wave * SPW + slot;
  uint4 krow[RW], vrow[RW];
  uint4 CS[NPL][QW];
  auto load_rows = [&](int base, int& jj) {
    const int it = base + my;
    jj = tok_lo + (it < n_tok ? it : n_tok - 1);   // always a real row
    const uint4* kr = reinterpret_cast<const uint4*>(a.kidx + (irow0 + jj) * CPT);
    const uint4* vr = reinterpret_cast<const uint4*>(a.vidx + (irow0 + jj) * CPT);
#pragma unroll
    for (int u = 0; u < RW; ++u) {
      krow[u] = kr[u];
      vrow[u] = vr[u];
    }
  };
  if (n_tok > 0) {
    int jj;
    load_rows(0, jj);
    load_cs(a.n_s + jj, CS);
  }
  int since_flush = 0;
  for (int base = 0; base < n_tok; base += NW * SPW) {
    const bool valid = base + my < n_tok;
    uint32_t ka[NCW], va[NCW];
    {
      uint32_t kd[4 * RW], vd[4 * RW];
#pragma unroll
      for (int u = 0; u < RW; ++u) {
        kd[4 * u] = krow[u].x; kd[4 * u + 1] = krow[u].y; kd[4 * u + 2] = krow[u].z; kd[4 * u + 3] = krow[u].w;
        vd[4 * u] = vrow[u].x; vd[4 * u + 1] = vrow[u].y; vd[4 * u + 2] = vrow[u].z; vd[4 * u + 3] = vrow[u].w;
      }
#pragma unroll
      for (int c = 0; c < NCW; ++c) {
        // chunk g + 4c (c < NPL) or the RoPE partner g + 4(c - NPL) + NP is byte g of word c
        ka[c] = __builtin_amdgcn_ubfe(kd[c], 8 * g, 8);
        va[c] = __builtin_amdgcn_ubfe(vd[c], 8 * g, 8);
      }
    }
    // Unconditional (clamped) next loads keep the prefetch in place without copies.
    int jn;
    load_rows(base + NW * SPW, jn);
    uint32_t Kw[NCW][C], Vw[NCW][C];
#pragma unroll
    for (int c = 0; c < NCW; ++c) gather(s_k, ka[c], Kw[c]);
#pragma unroll
    for (int c = 0; c < NCW; ++c) gather(s_v, va[c], Vw[c]);
    float sc[2];
    scores(Kw, CS, sc);
    load_cs(a.n_s + jn, CS);
    accumulate(sc, Vw, valid);
    if (++since_flush == kFlush) {
      flush();
      since_flush = 0;
    }
  }
  flush();

  // ---- merge the 8 slots of the wave (lanes with equal sl)
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
    for (int ml = 0; ml < 2; ++ml) {
      const float om = __shfl_xor(mrow[ml], off);
      const float ol = __shfl_xor(lrow[ml], off);
      const float mm = fmaxf(mrow[ml], om);
      const float a1 = mrow[ml] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrow[ml] - mm);
      const float a2 = om == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(om - mm);
      lrow[ml] = lrow[ml] * a1 + ol * a2;
#pragma unroll
      for (int k = 0; k < NPL; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int c = 0; c < C; ++c) {
            const float oa = __shfl_xor(acc[ml][k][p][c], off);
            acc[ml][k][p][c] = acc[ml][k][p][c] * a1 + oa * a2;
          }
      mrow[ml] = mm;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int ml = 0; ml < 2; ++ml) {
      const int m = 2 * hs + ml;
#pragma unroll
      for (int k = 0; k < NPL; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int c = 0; c < C; ++c) s_red[wave][m][p * HD + C * (g + 4 * k) + c] = acc[ml][k][p][c];
      if (g == 0) {
        s_red[wave][m][D] = mrow[ml];
        s_red[wave][m][D + 1] = lrow[ml];
      }
    }
  }
  __syncthreads();
  const float osc = ldexpf(1.f, shv);
  for (int x = tid; x < TC * D; x += kDecodeThreads) {
    const int m = x / D, d = x - m * D;
    const int t = beta * TC + m;
    if (t < t_lo || t >= t_hi) continue;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, s_red[w][m][D]);
    float num = 0.f, den = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = s_red[w][m][D];
        const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mm);
        num += f * s_red[w][m][d];
        den += f * s_red[w][m][D + 1];
      }
    }
    float* dst = a.ws + ((((int64_t)b * a.Hq + hq) * a.n_steps + (t - a.step0)) * a.n_split + split) * (D + 1);
    dst[d] = den > 0.f ? num / den * osc : 0.f;
    if (d == 0) dst[D] = den > 0.f ? (mm + __log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
}

// Single-step variant: one workgroup serves one loop step of one (batch,
// kv-head) for HPW q-heads of its GQA group.  Only the served step's slice of
// each codeword is staged (C fp16 per entry) and the eight lanes of a token
// split the channels, so no work is spent on the other steps of the block,
// and the codeword gathers and the RoPE rotation of a key are shared by the
// HPW heads.  Lane (g4, s2) owns the chunk pairs (q, q + D/(2c)) for
// q = g4 + 4 (s2 + 2k).  Used for per-step calls (n_steps = 1, the review's
// own per-step use) with one q-head per workgroup (GQA groups of two or four
// take the MFMA kernel of decode_gqa.hip).
template <int C, int HPW>
__global__ __launch_bounds__(kDecodeThreads) void decode_step_kernel(DecodeArgs a) {
  constexpr int D = 128, HD = 64, TC = 4, G = C * TC, CPT = D / C;
  constexpr int NP = HD / C;          // RoPE chunk pairs per token (16 or 8)
  constexpr int NPL = NP / 8;         // chunk pairs per lane (2 or 1)
  constexpr int DW = C / 2;           // dwords of one step of a codeword
  constexpr int QW = C / 4;           // sin/cos quads per chunk
  constexpr int RW = CPT / 16;        // uint4 per index row
  constexpr int PO = NP / 8;          // word-pair offset of the RoPE partner chunks
  constexpr int LPT = 8, SPW = kWave / LPT, NW = kDecodeThreads / kWave;
  __shared__ __attribute__((aligned(16))) uint32_t s_k[256 * DW];
  __shared__ __attribute__((aligned(16))) uint32_t s_v[256 * DW];
  __shared__ float s_red[NW][HPW][D + 2];
  __shared__ float s_amax[3][NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sl = lane & 7, slot = lane >> 3;
  const int g4 = sl & 3, s2 = sl >> 2;
  const int split = blockIdx.x;
  const int hq0 = blockIdx.y * HPW;   // first q-head served (HPW divides the GQA group)
  const int h = hq0 / a.gqa;
  const int b = blockIdx.z / a.n_steps;
  const int tl = blockIdx.z - b * a.n_steps;   // step within the served range
  const int t = a.step0 + tl;
  const int beta = t / TC, m = t - beta * TC;

  // ---- step m of both codebooks -> LDS (fp16), power-of-two range scaling
  const int64_t cbo = ((int64_t)h * a.n_blk + beta) * a.K * G;
  const int r = tid;   // one row per thread
  float kx[C], vx[C];
  float mq, mk, mv;   // the bf16 sinks and recent rows share the codebooks' scales
  decode_input_absmax(a, b, hq0, HPW, h, t, t + 1, split == 0, nullptr, mq, mk, mv);
#pragma unroll
  for (int i = 0; i < C; ++i) kx[i] = vx[i] = 0.f;
  if (r < a.K) {
#pragma unroll
    for (int i = 0; i < C; ++i) {
      // joint coordinate of channel i at step m is i*T_c + m
      kx[i] = bf16_to_f32(a.kcb[cbo + r * G + i * TC + m]);
      vx[i] = bf16_to_f32(a.vcb[cbo + r * G + i * TC + m]);
      mk = fmaxf(mk, fabsf(kx[i]));
      mv = fmaxf(mv, fabsf(vx[i]));
    }
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
  const int shk = pow2_range_shift(mk, 14), shv = pow2_range_shift(mv, kVLim), shq = pow2_range_shift(mq, 14);
  const float qsc = ldexpf(1.f, -shq);
  {
    const float sk = ldexpf(1.f, -shk), sv = ldexpf(1.f, -shv);
#pragma unroll
    for (int ip = 0; ip < DW; ++ip) {
      s_k[r * DW + ip] = pack_h2(kx[2 * ip] * sk, kx[2 * ip + 1] * sk);
      s_v[r * DW + ip] = pack_h2(vx[2 * ip] * sv, vx[2 * ip + 1] * sv);
    }
  }

  // ---- query words of the served heads: head hh, chunk pairs k, partner p, channel pair ip
  uint32_t qv[HPW][NPL][2][DW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    const uint16_t* qr = a.q + (((int64_t)b * a.Hq + hq0 + hh) * a.n_steps + tl) * D;
#pragma unroll
    for (int k = 0; k < NPL; ++k)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int d0 = p * HD + C * (g4 + 4 * (s2 + 2 * k));
#pragma unroll
        for (int ip = 0; ip < DW; ++ip) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(qr + d0 + 2 * ip);
          qv[hh][k][p][ip] = pack_h2(bf16lo(w) * qsc, bf16hi(w) * qsc);
        }
      }
  }
  const float sscale = a.qscale * ldexpf(1.f, shk + shq);

  float mrow[HPW], lrow[HPW];
  float acc[HPW][NPL][2][C];
  uint32_t acc16[HPW][NPL][2][DW];
#pragma unroll
  for (int hh = 0; hh < HPW; ++hh) {
    mrow[hh] = -INFINITY;
    lrow[hh] = 0.f;
#pragma unroll
    for (int k = 0; k < NPL; ++k)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int c = 0; c < C; ++c) acc[hh][k][p][c] = 0.f;
#pragma unroll
        for (int ip = 0; ip < DW; ++ip) acc16[hh][k][p][ip] = 0u;
      }
  }
  __syncthreads();

  int nb = a.N;
  if (a.seq_len) nb = max(0, min(a.seq_len[b], a.N));
  const int tok_lo = split * a.tok_per_split;
  const int tok_hi = min(nb, tok_lo + a.tok_per_split);
  const int n_sink = split == 0 ? a.n_s : 0;
  const int n_bf = n_sink + (split == 0 ? a.n_r : 0);
  const int64_t irow0 = (((int64_t)b * a.H + h) * a.n_blk + beta) * (int64_t)a.N_cap;
  const int64_t sink0 = (((int64_t)b * a.H + h) * a.T + t) * (int64_t)a.n_s;
  const int64_t rec0 = (((int64_t)b * a.H + h) * a.T + t) * (int64_t)a.r_cap;
  const uint16_t* rope16 = reinterpret_cast<const uint16_t*>(a.rope);
  const float ksc = ldexpf(1.f, -shk), vsc = ldexpf(1.f, -shv);

  // Kw[k] / Kw[NPL + k]: this step's words of chunk pair k and of its partner.
  // The key is rotated once and scored against every served head.
  auto scores = [&](const uint32_t (&Kw)[2 * NPL][DW], const uint4 (&CS)[NPL][QW], float (&sc)[HPW]) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) sc[hh] = 0.f;
#pragma unroll
    for (int k = 0; k < NPL; ++k)
#pragma unroll
      for (int ip = 0; ip < DW; ++ip) {
        const uint4 q4 = CS[k][ip >> 1];
        const h2_t c2 = as_h2((ip & 1) ? q4.y : q4.x), s2v = as_h2((ip & 1) ? q4.w : q4.z);
        const h2_t x1 = as_h2(Kw[k][ip]), x2 = as_h2(Kw[NPL + k][ip]);
        const h2_t r1 = x1 * c2 - x2 * s2v;
        const h2_t r2 = x2 * c2 + x1 * s2v;
#pragma unroll
        for (int hh = 0; hh < HPW; ++hh) {
          sc[hh] = __builtin_amdgcn_fdot2(r1, as_h2(qv[hh][k][0][ip]), sc[hh], false);
          sc[hh] = __builtin_amdgcn_fdot2(r2, as_h2(qv[hh][k][1][ip]), sc[hh], false);
        }
      }
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) sc[hh] = group_sum<8>(sc[hh]) * sscale;
  };
  auto flush = [&]() {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh)
#pragma unroll
      for (int k = 0; k < NPL; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int ip = 0; ip < DW; ++ip) {
            add_f16x2(acc16[hh][k][p][ip], acc[hh][k][p][2 * ip], acc[hh][k][p][2 * ip + 1]);
            acc16[hh][k][p][ip] = 0u;
          }
  };
  // Online softmax per head (base 2; the running maximum lags by at most
  // kLag) and P*V.
  auto accumulate = [&](const float (&sc)[HPW], const uint32_t (&Vw)[2 * NPL][DW], bool valid) {
    if (!valid) return;
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float s = sc[hh];
      if (s > mrow[hh] + (float)kLag) {
        const float alpha = __builtin_amdgcn_exp2f(mrow[hh] - s);
        const h2_t a2 = {(_Float16)alpha, (_Float16)alpha};
        lrow[hh] *= alpha;
#pragma unroll
        for (int k = 0; k < NPL; ++k)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
#pragma unroll
            for (int c = 0; c < C; ++c) acc[hh][k][p][c] *= alpha;
#pragma unroll
            for (int ip = 0; ip < DW; ++ip)
              acc16[hh][k][p][ip] = __builtin_bit_cast(uint32_t, as_h2(acc16[hh][k][p][ip]) * a2);
          }
        mrow[hh] = s;
      }
      const float pr = __builtin_amdgcn_exp2f(s - mrow[hh]);
      lrow[hh] += pr;
      const h2_t p2 = {(_Float16)pr, (_Float16)pr};
#pragma unroll
      for (int k = 0; k < NPL; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int ip = 0; ip < DW; ++ip) {
            const h2_t v2 = as_h2(Vw[p * NPL + k][ip]);
            acc16[hh][k][p][ip] = __builtin_bit_cast(uint32_t, v2 * p2 + as_h2(acc16[hh][k][p][ip]));
          }
    }
  };
  auto load_cs = [&](int pos, uint4 (&CS)[NPL][QW]) {
    const uint4* row = reinterpret_cast<const uint4*>(rope16 + (int64_t)pos * D);
#pragma unroll
    for (int k = 0; k < NPL; ++k)
#pragma unroll
      for (int u = 0; u < QW; ++u) CS[k][u] = row[QW * (g4 + 4 * (s2 + 2 * k)) + u];
  };

  // Sinks and the recent window (split 0 only), straight from the bf16 rows.
  for (int base = 0; base < n_bf; base += NW * SPW) {
    const int item = base + wave * SPW + slot;
    const bool valid = item < n_bf;
    const int it = valid ? item : 0;
    const bool is_rec = it >= n_sink;
    const int pos = is_rec ? a.n_s + nb + (it - n_sink) : it;
    const uint16_t* kr = is_rec ? a.rk + (rec0 + (it - n_sink)) * D : a.sk + (sink0 + it) * D;
    const uint16_t* vr = is_rec ? a.rv + (rec0 + (it - n_sink)) * D : a.sv + (sink0 + it) * D;
    uint32_t Kw[2 * NPL][DW], Vw[2 * NPL][DW];
#pragma unroll
    for (int c = 0; c < 2 * NPL; ++c) {
      const int k = c % NPL, p = c / NPL;
      const int d0 = p * HD + C * (g4 + 4 * (s2 + 2 * k));
#pragma unroll
      for (int ip = 0; ip < DW; ++ip) {
        const uint32_t x = *reinterpret_cast<const uint32_t*>(kr + d0 + 2 * ip);
        const uint32_t y = *reinterpret_cast<const uint32_t*>(vr + d0 + 2 * ip);
        Kw[c][ip] = pack_h2(bf16lo(x) * ksc, bf16hi(x) * ksc);
        Vw[c][ip] = pack_h2(bf16lo(y) * vsc, bf16hi(y) * vsc);
      }
    }
    uint4 CS[NPL][QW];
    load_cs(pos, CS);
    float sc[HPW];
    scores(Kw, CS, sc);
    accumulate(sc, Vw, valid);
    flush();
  }

  // Context tokens; index rows and sin/cos quads are prefetched one token ahead.
  // Index byte of chunk c is byte c % 4 of word c / 4; this lane's chunks sit
  // in word pairs (k, and k + PO for the partners) at byte 4*s2 + g4.
  const uint32_t psel = 0x0c0c0c00u | (uint32_t)(4 * s2 + g4);
  const int n_tok = max(0, tok_hi - tok_lo);
  const int my = wave * SPW + slot;
  uint4 krow[RW], vrow[RW];
  uint4 CS[NPL][QW];
  auto load_rows = [&](int base, int& jj) {
    const int it = base + my;
    jj = tok_lo + (it < n_tok ? it : n_tok - 1);   // always a real row
    const uint4* kr = reinterpret_cast<const uint4*>(a.kidx + (irow0 + jj) * CPT);
    const uint4* vr = reinterpret_cast<const uint4*>(a.vidx + (irow0 + jj) * CPT);
#pragma unroll
    for (int u = 0; u < RW; ++u) {
      krow[u] = kr[u];
      vrow[u] = vr[u];
    }
  };
  if (n_tok > 0) {
    int jj;
    load_rows(0, jj);
    load_cs(a.n_s + jj, CS);
  }
  int since_flush = 0;
  for (int base = 0; base < n_tok; base += NW * SPW) {
    const bool valid = base + my < n_tok;
    uint32_t kd[4 * RW], vd[4 * RW];
#pragma unroll
    for (int u = 0; u < RW; ++u) {
      kd[4 * u] = krow[u].x; kd[4 * u + 1] = krow[u].y; kd[4 * u + 2] = krow[u].z; kd[4 * u + 3] = krow[u].w;
      vd[4 * u] = vrow[u].x; vd[4 * u + 1] = vrow[u].y; vd[4 * u + 2] = vrow[u].z; vd[4 * u + 3] = vrow[u].w;
    }
    int jn;
    load_rows(base + NW * SPW, jn);
    uint32_t Kw[2 * NPL][DW], Vw[2 * NPL][DW];
#pragma unroll
    for (int c = 0; c < 2 * NPL; ++c) {
      const int wp = (c % NPL) + (c / NPL) * PO;     // word pair of chunk c
      const uint32_t ik = __builtin_amdgcn_perm(kd[2 * wp + 1], kd[2 * wp], psel);
      const uint32_t iv = __builtin_amdgcn_perm(vd[2 * wp + 1], vd[2 * wp], psel);
      if constexpr (DW == 2) {
        const uint2 x = *reinterpret_cast<const uint2*>(&s_k[ik * DW]);
        const uint2 y = *reinterpret_cast<const uint2*>(&s_v[iv * DW]);
        Kw[c][0] = x.x; Kw[c][1] = x.y;
        Vw[c][0] = y.x; Vw[c][1] = y.y;
      } else {
        const uint4 x = *reinterpret_cast<const uint4*>(&s_k[ik * DW]);
        const uint4 y = *reinterpret_cast<const uint4*>(&s_v[iv * DW]);
        Kw[c][0] = x.x; Kw[c][1] = x.y; Kw[c][2] = x.z; Kw[c][3] = x.w;
        Vw[c][0] = y.x; Vw[c][1] = y.y; Vw[c][2] = y.z; Vw[c][3] = y.w;
      }
    }
    float sc[HPW];
    scores(Kw, CS, sc);
    load_cs(a.n_s + jn, CS);
    accumulate(sc, Vw, valid);
    if (++since_flush == kFlush) {
      flush();
      since_flush = 0;
    }
  }
  flush();

  // ---- merge the 8 slots of the wave (lanes with equal sl), then the waves
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
      const float om = __shfl_xor(mrow[hh], off);
      const float ol = __shfl_xor(lrow[hh], off);
      const float mm = fmaxf(mrow[hh], om);
      const float a1 = mrow[hh] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrow[hh] - mm);
      const float a2 = om == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(om - mm);
      lrow[hh] = lrow[hh] * a1 + ol * a2;
#pragma unroll
      for (int k = 0; k < NPL; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int c = 0; c < C; ++c) {
            const float oa = __shfl_xor(acc[hh][k][p][c], off);
            acc[hh][k][p][c] = acc[hh][k][p][c] * a1 + oa * a2;
          }
      mrow[hh] = mm;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int hh = 0; hh < HPW; ++hh) {
#pragma unroll
      for (int k = 0; k < NPL; ++k)
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
          for (int c = 0; c < C; ++c)
            s_red[wave][hh][p * HD + C * (g4 + 4 * (s2 + 2 * k)) + c] = acc[hh][k][p][c];
      if (sl == 0) {
        s_red[wave][hh][D] = mrow[hh];
        s_red[wave][hh][D + 1] = lrow[hh];
      }
    }
  }
  __syncthreads();
  const float osc = ldexpf(1.f, shv);
  for (int x = tid; x < HPW * D; x += kDecodeThreads) {
    const int hh = x / D, d = x - hh * D;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, s_red[w][hh][D]);
    float num = 0.f, den = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = s_red[w][hh][D];
        const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mm);
        num += f * s_red[w][hh][d];
        den += f * s_red[w][hh][D + 1];
      }
    }
    float* dst = a.ws + ((((int64_t)b * a.Hq + hq0 + hh) * a.n_steps + tl) * a.n_split + split) * (D + 1);
    dst[d] = den > 0.f ? num / den * osc : 0.f;
    if (d == 0) dst[D] = den > 0.f ? (mm + __log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
}

hipError_t launch_decode_fast(int G, const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.Hq, a.B * a.n_blk_serv);
  if (G == 16)
    return launch_decode_half(a, s);   // one-instruction index decode (decode_half.hip)
  else if (G == 32)
    hipLaunchKernelGGL(decode_fast_kernel<8>, grid, dim3(kDecodeThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_step(int G, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.n_split, a.Hq, a.B * a.n_steps);
  if (G == 16)
    hipLaunchKernelGGL((decode_step_kernel<4, 1>), grid, dim3(kDecodeThreads), 0, s, a);
  else if (G == 32)
    hipLaunchKernelGGL((decode_step_kernel<8, 1>), grid, dim3(kDecodeThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace loopvq
