// LoopVQ fused decode attention for GQA groups of four q-heads over blocks of
// four loop steps (T_c = 4, c = 4 or 8, no pre-transform).
//
// LoopVQ review (arXiv 2611.05304), section 3.4 step 3 (codebook on chip,
// lookup by index, RoPE from a precomputed table after dequant, Flash-
// Decoding split merge) and section 3.1 eq. (5) (step m reads coordinate
// i*T_c + m of the shared codeword).
//
// Four q-heads x four steps give 16 score rows per token, so the scores are a
// real contraction and run on v_mfma_f32_16x16x32_f16: rows (h, m) = 4h + m,
// columns = 16 tokens, k = 128 channels in four blocks of 32.  The keys of
// step m go through their own chain of four MFMAs whose rows of step m are
// kept (the other rows pair a query with another step's keys and are
// dropped).  Each wave works on 16 tokens at a time and plays two roles:
//   * score lanes (token t = lane % 16, quarter q4 = lane / 16): gather the
//     token's K codewords of the chunks holding channels 32r + 8q4 + j,
//     rotate them (their RoPE partners are in the same lane) straight into the
//     MFMA B operand, and receive the scores of head q4 for the four steps;
//     they keep the online softmax of those rows (the running maximum is
//     shared by the 16 token lanes of a row through DPP).
//   * P.V lanes (channel group cg = lane % 16, step m = lane / 16): own the
//     output of channels 8cg .. 8cg+7 at step m for the four heads; per token
//     they gather the V codeword slice themselves and read the four
//     probabilities from a per-wave LDS tile.
// Every index byte is used once for K and once for V per token, every
// codeword gather and key rotation serves all four heads.
#include "common.h"
#include "kernels.h"

namespace loopvq {

namespace {

typedef _Float16 h2g_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4g_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2g_t as_h2g(uint32_t w) { return __builtin_bit_cast(h2g_t, w); }

__device__ __forceinline__ uint32_t pack_h2g(float a, float b) {
  const _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

__device__ __forceinline__ int pow2_shift_g(float max_abs, int lim) {
  if (!(max_abs > 0.f)) return 0;
  const int e = ilogbf(max_abs) + 1;
  return e > lim ? e - lim : 0;
}

// max over the 16 lanes of a DPP row
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, true)));
  return v;
}

// Orders this wave's LDS traffic: writes before the fence are visible to the
// wave's reads after it.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kGLag = 3, kGVLim = 7;   // running-max lag and value range, as in the other decode kernels

}  // namespace

template <int C>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_gqa_kernel(DecodeArgs a) {
  constexpr int D = 128, HD = 64, TC = 4, G = C * TC, CPT = D / C;
  constexpr int CW = G / 8;           // uint4 per codeword (fp16, step-major)
  // Codeword stride in uint4: one pad slot makes it odd, so the step-m slices
  // of random codewords spread over all LDS bank groups (a stride of 4 slots
  // would put every step-m read of a wave in the same 4 of 16 groups).
  constexpr int CWS = CW + 1;
  constexpr int DW = C / 2;           // dwords of one step of a codeword
  constexpr int RW = CPT / 16;        // uint4 per index row
  constexpr int NW = kDecodeThreads / kWave;
  constexpr int TOK = 16;             // tokens per wave iteration
  // K and V codebooks; after the token loops the same memory holds the
  // per-wave partial rows of the final merge.
  constexpr int KV_U4 = 2 * 256 * CWS, RED_U4 = (NW * 16 * (D + 2) * 4 + 15) / 16;
  __shared__ __attribute__((aligned(16))) uint4 s_kv[KV_U4 > RED_U4 ? KV_U4 : RED_U4];
  uint4* const s_k = s_kv;
  uint4* const s_v = s_kv + 256 * CWS;
  float (*const s_red)[16][D + 2] = reinterpret_cast<float (*)[16][D + 2]>(s_kv);
  __shared__ __attribute__((aligned(16))) uint32_t s_p[NW][TOK][4][4];      // [t][m][h] fp16 pairs (p, p)
  __shared__ float s_alpha[NW][4][4];                                        // [m][h]
  __shared__ __attribute__((aligned(16))) uint8_t s_vix[NW][CPT][TOK];      // V index bytes, transposed
  __shared__ float s_amax[2][NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t16 = lane & 15, q4 = lane >> 4;     // score role: token, quarter (= head)
  const int cg = lane & 15, ms = lane >> 4;      // P.V role: channel group, step
  const int split = blockIdx.x;
  const int hq0 = blockIdx.y * 4;
  const int h = hq0 / a.gqa;
  const int b = blockIdx.z / a.n_blk_serv;
  const int beta = a.blk0 + (blockIdx.z - b * a.n_blk_serv);
  const int t_lo = max(a.step0, beta * TC), t_hi = min(a.step0 + a.n_steps, (beta + 1) * TC);

  // ---- codebooks -> LDS (fp16, step-major), power-of-two range scaling
  const int64_t cbo = ((int64_t)h * a.n_blk + beta) * a.K * G;
  const int r = tid;
  float kx[G], vx[G];
  float mk = 0.f, mv = 0.f;
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
    mk = fmaxf(mk, __shfl_xor(mk, off));
    mv = fmaxf(mv, __shfl_xor(mv, off));
  }
  if (lane == 0) {
    s_amax[0][wave] = mk;
    s_amax[1][wave] = mv;
  }
  __syncthreads();
  mk = fmaxf(fmaxf(s_amax[0][0], s_amax[0][1]), fmaxf(s_amax[0][2], s_amax[0][3]));
  mv = fmaxf(fmaxf(s_amax[1][0], s_amax[1][1]), fmaxf(s_amax[1][2], s_amax[1][3]));
  const int shk = pow2_shift_g(mk, 14), shv = pow2_shift_g(mv, kGVLim);
  {
    const float sk = ldexpf(1.f, -shk), sv = ldexpf(1.f, -shv);
    uint32_t kw[TC * DW], vw[TC * DW];   // [m][channel pair]
#pragma unroll
    for (int m = 0; m < TC; ++m)
#pragma unroll
      for (int ip = 0; ip < DW; ++ip) {
        kw[m * DW + ip] = pack_h2g(kx[(2 * ip) * TC + m] * sk, kx[(2 * ip + 1) * TC + m] * sk);
        vw[m * DW + ip] = pack_h2g(vx[(2 * ip) * TC + m] * sv, vx[(2 * ip + 1) * TC + m] * sv);
      }
#pragma unroll
    for (int u = 0; u < CW; ++u) {
      s_k[r * CWS + u] = make_uint4(kw[4 * u], kw[4 * u + 1], kw[4 * u + 2], kw[4 * u + 3]);
      s_v[r * CWS + u] = make_uint4(vw[4 * u], vw[4 * u + 1], vw[4 * u + 2], vw[4 * u + 3]);
    }
  }

  // ---- query operand: row rho = lane % 16 = (head rho/4, step rho%4), k quarter
  // kq = lane / 16; block r' holds channels 32r' + 8kq .. +7 of the row's step.
  h8_t qa[4];
  {
    const int rho = lane & 15, kq = lane >> 4;
    const int hh = rho >> 2, m = rho & 3;
    const int t = beta * TC + m;
    const bool act = t >= t_lo && t < t_hi;
    const uint16_t* qr = a.q + (((int64_t)b * a.Hq + hq0 + hh) * a.n_steps + (act ? t - a.step0 : 0)) * D;
#pragma unroll
    for (int rp = 0; rp < 4; ++rp) {
      const uint4 w = *reinterpret_cast<const uint4*>(qr + 32 * rp + 8 * kq);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qa[rp][2 * e] = act ? (_Float16)bf16lo(ws[e]) : (_Float16)0.f;
        qa[rp][2 * e + 1] = act ? (_Float16)bf16hi(ws[e]) : (_Float16)0.f;
      }
    }
  }
  const float sscale = a.qscale * ldexpf(1.f, shk);

  // score-role state: rows (head q4, step i)
  float Mr[TC], Lr[TC];
#pragma unroll
  for (int i = 0; i < TC; ++i) {
    Mr[i] = -INFINITY;
    Lr[i] = 0.f;
  }
  // P.V-role state: heads hh, channels 8cg + 2ip, +1 of step ms
  float acc[4][8];
  uint32_t acc16[4][4];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
#pragma unroll
  for (int hh = 0; hh < 4; ++hh)
#pragma unroll
    for (int ip = 0; ip < 4; ++ip) acc16[hh][ip] = 0u;
  __syncthreads();

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

  // Score lane data of one token: Kc[m][r'] = 8 channels 32r' + 8q4 .. +7 of
  // step m as four fp16 pairs (before rotation).  cos/sin: quads 8r + 2q4 and
  // 8r + 2q4 + 1 for r in {0, 1} (frequencies 32r + 8q4 .. +7).
  // One accumulator chain per key step m: row (h, m') of chain m holds the
  // score of q-head h at step m' against the keys of step m, so a lane keeps
  // element i of chain i (rows 4q4 + i are (head q4, step i)).
  auto rotate_score = [&](uint32_t (&Kc)[TC][4][4], const uint4 (&CS)[2][2], bool valid, float (&s)[TC]) {
#pragma unroll
    for (int m = 0; m < TC; ++m) {
      f4g_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rr = 0; rr < 2; ++rr) {
        uint32_t o1[4], o2[4];
#pragma unroll
        for (int ip = 0; ip < 4; ++ip) {
          const uint4 q = CS[rr][ip >> 1];
          const h2g_t c2 = as_h2g((ip & 1) ? q.y : q.x), s2 = as_h2g((ip & 1) ? q.w : q.z);
          const h2g_t x1 = as_h2g(Kc[m][rr][ip]), x2 = as_h2g(Kc[m][rr + 2][ip]);
          o1[ip] = __builtin_bit_cast(uint32_t, x1 * c2 - x2 * s2);
          o2[ip] = __builtin_bit_cast(uint32_t, x2 * c2 + x1 * s2);
        }
        const h8_t b1 = __builtin_bit_cast(h8_t, make_uint4(o1[0], o1[1], o1[2], o1[3]));
        const h8_t b2 = __builtin_bit_cast(h8_t, make_uint4(o2[0], o2[1], o2[2], o2[3]));
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[rr], b1, sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[rr + 2], b2, sacc, 0, 0, 0);
      }
      s[m] = valid ? sacc[m] * sscale : -INFINITY;
    }
  };

  // Softmax of the score rows, then the P tile and the rescale factors go to
  // this wave's LDS slots.  Returns true when some row's maximum moved.
  auto softmax_tile = [&](const float (&s)[TC]) {
    bool moved = false;
#pragma unroll
    for (int i = 0; i < TC; ++i) {
      const float mx = row16_max(s[i]);
      float alpha = 1.f;
      if (mx > Mr[i] + (float)kGLag) {
        alpha = Mr[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mr[i] - mx);
        Mr[i] = mx;
        Lr[i] *= alpha;
        moved = true;
      }
      const float p = Mr[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[i] - Mr[i]);
      Lr[i] += p;
      const _Float16 ph = (_Float16)p;
      s_p[wave][t16][i][q4] = (uint32_t)__builtin_bit_cast(uint16_t, ph) * 0x10001u;
      if (t16 == 0) s_alpha[wave][i][q4] = alpha;
    }
    return __ballot(moved) != 0;
  };

  // P.V of one token slot for this lane's (channel group, step); Vw = the
  // four fp16 pairs of channels 8cg .. 8cg+7 at step ms.
  auto pv = [&](int t, const uint32_t (&Vw)[4]) {
    const uint4 p4 = *reinterpret_cast<const uint4*>(&s_p[wave][t][ms][0]);
    const uint32_t pw[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
    for (int hh = 0; hh < 4; ++hh)
#pragma unroll
      for (int ip = 0; ip < 4; ++ip)
        acc16[hh][ip] = __builtin_bit_cast(uint32_t, as_h2g(Vw[ip]) * as_h2g(pw[hh]) + as_h2g(acc16[hh][ip]));
  };
  auto rescale = [&]() {
    const float4 al = *reinterpret_cast<const float4*>(&s_alpha[wave][ms][0]);
    const float alv[4] = {al.x, al.y, al.z, al.w};
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const h2g_t a2 = {(_Float16)alv[hh], (_Float16)alv[hh]};
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[hh][e] *= alv[hh];
#pragma unroll
      for (int ip = 0; ip < 4; ++ip) acc16[hh][ip] = __builtin_bit_cast(uint32_t, as_h2g(acc16[hh][ip]) * a2);
    }
  };
  auto flush = [&]() {
#pragma unroll
    for (int hh = 0; hh < 4; ++hh)
#pragma unroll
      for (int ip = 0; ip < 4; ++ip) {
        add_f16x2(acc16[hh][ip], acc[hh][2 * ip], acc[hh][2 * ip + 1]);
        acc16[hh][ip] = 0u;
      }
  };
  auto load_cs = [&](int pos, uint4 (&CS)[2][2]) {
    const uint4* row = reinterpret_cast<const uint4*>(rope16 + (int64_t)pos * D);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int u = 0; u < 2; ++u) CS[rr][u] = row[8 * rr + 2 * q4 + u];
  };

  // ---- bf16 items: sinks at positions 0..n_s-1, then the recent window at
  // n_s + N_b + r (split 0 only), 16 per wave iteration
  for (int base = 0; base < n_bf; base += NW * TOK) {
    // score role: item base + 16*wave + t16
    {
      const int item = base + wave * TOK + t16;
      const bool valid = item < n_bf;
      const int it = valid ? item : 0;
      const bool is_rec = it >= n_sink;
      const int pos = is_rec ? a.n_s + nb + (it - n_sink) : it;
      uint32_t Kc[TC][4][4];
#pragma unroll
      for (int m = 0; m < TC; ++m) {
        const uint16_t* kr = is_rec ? a.rk + (rec0 + (int64_t)m * a.r_cap + (it - n_sink)) * D
                                    : a.sk + (sink0 + (int64_t)m * a.n_s + it) * D;
#pragma unroll
        for (int rp = 0; rp < 4; ++rp) {
          const uint4 w = *reinterpret_cast<const uint4*>(kr + 32 * rp + 8 * q4);
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) Kc[m][rp][e] = pack_h2g(bf16lo(ws[e]) * ksc, bf16hi(ws[e]) * ksc);
        }
      }
      uint4 CS[2][2];
      load_cs(pos, CS);
      float s[TC];
      rotate_score(Kc, CS, valid, s);
      const bool moved = softmax_tile(s);
      wave_sync();
      if (moved) rescale();
    }
    // P.V role: the same 16 items, channels 8cg .. 8cg+7 of step ms
#pragma unroll 1
    for (int t = 0; t < TOK; ++t) {
      const int item = base + wave * TOK + t;
      const int it = item < n_bf ? item : 0;
      const bool is_rec = it >= n_sink;
      const uint16_t* vr = is_rec ? a.rv + (rec0 + (int64_t)ms * a.r_cap + (it - n_sink)) * D
                                  : a.sv + (sink0 + (int64_t)ms * a.n_s + it) * D;
      const uint4 w = *reinterpret_cast<const uint4*>(vr + 8 * cg);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      uint32_t Vw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) Vw[e] = pack_h2g(bf16lo(ws[e]) * vsc, bf16hi(ws[e]) * vsc);
      pv(t, Vw);   // p = 0 for items past the end
    }
    flush();
    wave_sync();
  }

  // ---- quantized tokens: 16 per wave iteration, index rows prefetched
  const int n_tok = max(0, tok_hi - tok_lo);
  uint4 krow[RW], vrow[RW];
  uint4 CS[2][2];
  auto load_rows = [&](int base, int& jj) {
    const int it = base + wave * TOK + t16;
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
  int tiles = 0;
  for (int base = 0; base < n_tok; base += NW * TOK) {
    const bool valid = base + wave * TOK + t16 < n_tok;
    uint32_t kd[4 * RW], vd[4 * RW];
#pragma unroll
    for (int u = 0; u < RW; ++u) {
      kd[4 * u] = krow[u].x; kd[4 * u + 1] = krow[u].y; kd[4 * u + 2] = krow[u].z; kd[4 * u + 3] = krow[u].w;
      vd[4 * u] = vrow[u].x; vd[4 * u + 1] = vrow[u].y; vd[4 * u + 2] = vrow[u].z; vd[4 * u + 3] = vrow[u].w;
    }
    // V index bytes of this quarter's chunks, transposed for the P.V lanes:
    // s_vix[c][t] for c in [q4 * CPT/4, (q4 + 1) * CPT/4).
#pragma unroll
    for (int e = 0; e < CPT / 4; ++e) {
      const int c = q4 * (CPT / 4) + e;
      s_vix[wave][c][t16] = (uint8_t)__builtin_amdgcn_ubfe(vd[c >> 2], 8 * (c & 3), 8);
    }
    int jn;
    load_rows(base + NW * TOK, jn);
    // K codewords of the chunks holding channels 32r + 8q4 + j (j < 8)
    uint32_t Kc[TC][4][4];
#pragma unroll
    for (int rp = 0; rp < 4; ++rp) {
      if constexpr (C == 8) {
        const int c = 4 * rp + q4;                          // chunk = channels 8c .. 8c+7
        const uint32_t ik = __builtin_amdgcn_ubfe(kd[c >> 2], 8 * (c & 3), 8);
        const uint4* cw = &s_k[ik * CWS];
#pragma unroll
        for (int m = 0; m < TC; ++m) {
          const uint4 x = cw[m];                            // step m: 8 channels
          Kc[m][rp][0] = x.x; Kc[m][rp][1] = x.y; Kc[m][rp][2] = x.z; Kc[m][rp][3] = x.w;
        }
      } else {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int c = 8 * rp + 2 * q4 + half;             // chunk = channels 4c .. 4c+3
          const uint32_t ik = __builtin_amdgcn_ubfe(kd[c >> 2], 8 * (c & 3), 8);
          const uint4* cw = &s_k[ik * CWS];
          const uint4 x0 = cw[0], x1 = cw[1];               // steps 0-1, 2-3
          Kc[0][rp][2 * half] = x0.x; Kc[0][rp][2 * half + 1] = x0.y;
          Kc[1][rp][2 * half] = x0.z; Kc[1][rp][2 * half + 1] = x0.w;
          Kc[2][rp][2 * half] = x1.x; Kc[2][rp][2 * half + 1] = x1.y;
          Kc[3][rp][2 * half] = x1.z; Kc[3][rp][2 * half + 1] = x1.w;
        }
      }
    }
    float s[TC];
    rotate_score(Kc, CS, valid, s);
    load_cs(a.n_s + jn, CS);
    const bool moved = softmax_tile(s);
    wave_sync();
    if (moved) rescale();
    // P.V lanes: V index bytes of chunk(s) of this channel group for the 16 tokens
    if constexpr (C == 8) {
      const uint4 ix = *reinterpret_cast<const uint4*>(&s_vix[wave][cg][0]);
      const uint32_t iw[4] = {ix.x, ix.y, ix.z, ix.w};
#pragma unroll
      for (int t = 0; t < TOK; ++t) {
        const uint32_t iv = __builtin_amdgcn_ubfe(iw[t >> 2], 8 * (t & 3), 8);
        const uint4 y = s_v[iv * CWS + ms];
        const uint32_t Vw[4] = {y.x, y.y, y.z, y.w};
        pv(t, Vw);
      }
    } else {
      const uint4 ia = *reinterpret_cast<const uint4*>(&s_vix[wave][2 * cg][0]);
      const uint4 ib = *reinterpret_cast<const uint4*>(&s_vix[wave][2 * cg + 1][0]);
      const uint32_t wa[4] = {ia.x, ia.y, ia.z, ia.w}, wb[4] = {ib.x, ib.y, ib.z, ib.w};
#pragma unroll
      for (int t = 0; t < TOK; ++t) {
        const uint32_t va = __builtin_amdgcn_ubfe(wa[t >> 2], 8 * (t & 3), 8);
        const uint32_t vb = __builtin_amdgcn_ubfe(wb[t >> 2], 8 * (t & 3), 8);
        // step ms of a 4-channel codeword: dwords 2ms, 2ms+1
        const uint2 ya = reinterpret_cast<const uint2*>(&s_v[va * CWS])[ms];
        const uint2 yb = reinterpret_cast<const uint2*>(&s_v[vb * CWS])[ms];
        const uint32_t Vw[4] = {ya.x, ya.y, yb.x, yb.y};
        pv(t, Vw);
      }
    }
    // fp16 partials over two tiles (32 tokens): |p| <= 2^kGLag, |v| <= 2^kGVLim,
    // so a partial stays below 2^15
    if (++tiles == 2) {
      flush();
      tiles = 0;
    }
    wave_sync();
  }
  flush();

  // ---- per-wave row totals, then merge the waves through LDS (the codebook
  // memory, once every wave is done with it)
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TC; ++i) {
    float l = Lr[i];
    l += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(l), 0xB1, 0xF, 0xF, true));
    l += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(l), 0x4E, 0xF, 0xF, true));
    l += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(l), 0x141, 0xF, 0xF, true));
    l += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(l), 0x140, 0xF, 0xF, true));
    if (t16 == 0) {
      s_red[wave][4 * q4 + i][D] = Mr[i];
      s_red[wave][4 * q4 + i][D + 1] = l;
    }
  }
#pragma unroll
  for (int hh = 0; hh < 4; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) s_red[wave][4 * hh + ms][8 * cg + e] = acc[hh][e];
  __syncthreads();
  const float osc = ldexpf(1.f, shv);
  for (int x = tid; x < 16 * D; x += kDecodeThreads) {
    const int rho = x / D, d = x - rho * D;
    const int hh = rho >> 2, m = rho & 3;
    const int t = beta * TC + m;
    if (t < t_lo || t >= t_hi) continue;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, s_red[w][rho][D]);
    float num = 0.f, den = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = s_red[w][rho][D];
        const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mm);
        num += f * s_red[w][rho][d];
        den += f * s_red[w][rho][D + 1];
      }
    }
    float* dst = a.ws + ((((int64_t)b * a.Hq + hq0 + hh) * a.n_steps + (t - a.step0)) * a.n_split + split) * (D + 1);
    dst[d] = den > 0.f ? num / den * osc : 0.f;
    if (d == 0) dst[D] = den > 0.f ? (mm + __log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
}

hipError_t launch_decode_gqa(int G, const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.Hq / 4, a.B * a.n_blk_serv);
  if (G == 16)
    hipLaunchKernelGGL(decode_gqa_kernel<4>, grid, dim3(kDecodeThreads), 0, s, a);
  else if (G == 32)
    hipLaunchKernelGGL(decode_gqa_kernel<8>, grid, dim3(kDecodeThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace loopvq
