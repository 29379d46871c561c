// LoopVQ fused decode attention for GQA groups of two or four q-heads over
// blocks of four loop steps (T_c = 4, c = 4 or 8, no pre-transform).
//
// LoopVQ review (arXiv 2611.05304), section 3.4 step 3 (codebook on chip,
// lookup by index, RoPE from a precomputed table after dequant, Flash-
// Decoding split merge) and section 3.1 eq. (5) (step m reads coordinate
// i*T_c + m of the shared codeword).
//
// Four q-heads x four steps give 16 rows rho = 4h + m per token, so both
// products are real contractions and run on v_mfma_f32_16x16x32_f16 (a
// workgroup may also serve a group of two q-heads: the rows of heads 2 and 3
// then carry zero queries and are not written):
//   * scores S^T[token][rho] (A = rotated keys of 16 tokens, B = queries,
//     k = 128 channels in four blocks of 32).  The keys of step m go through
//     their own chain of MFMAs; a lane keeps the chain of its row's step.
//     Key lanes (token t16 = lane % 16, quarter q4 = lane / 16) gather the
//     token's K codewords of the chunks holding channels 32r + 8q4 + j and
//     rotate them (RoPE partners sit in the same lane) into the A operand.
//   * row lanes (rho = lane % 16, group g = lane / 16) receive the scores of
//     row rho for tokens 4g .. 4g+3 of each 16-token tile, keep the row's
//     online softmax (the maximum crosses the four groups through permlane
//     swaps) and hold the row's output O^T[channel][rho] for channels
//     16b + 4g .. +3 of every 16-channel block b.
//   * P.V: O^T += V_m^T P_m per step m, with P_m = P masked to the rows of
//     step m and V_m^T [16 channels][32 tokens] read straight from the LDS
//     codebook by ds_read_b64_tr_b16: within a 16-lane group, lane (a, j)
//     fetches four channels 4a .. 4a+3 of token j, and the transposed read
//     hands every lane one channel of four tokens.
// Every index byte is used once for K and once for V per token; every
// codeword gather and key rotation serves all four heads.  With a single
// served step (ONE) only that step's key slices are gathered and rotated, one
// score chain runs and P needs no step mask.
#include "common.h"
#include "kernels.h"

namespace loopvq {

namespace {

typedef _Float16 h2g_t __attribute__((ext_vector_type(2)));
typedef _Float16 h4g_t __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4g_t __attribute__((ext_vector_type(4)));
typedef short s4g_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4g_t lds_s4_t;

__device__ __forceinline__ h2g_t as_h2g(uint32_t w) { return __builtin_bit_cast(h2g_t, w); }

__device__ __forceinline__ uint32_t pack_h2g(float a, float b) {
  const _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// Four fp16 at an 8-byte aligned LDS byte address, transposed within the
// lane's 16-lane group (ds_read_b64_tr_b16).
__device__ __forceinline__ h4g_t lds_tr4(const void* base, uint32_t byte_off) {
  return __builtin_bit_cast(h4g_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s4_t*)((__attribute__((address_space(3))) char*)(__attribute__((address_space(3))) void*)base + byte_off)));
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

template <int C, int HPW, bool ONE>
__global__ __launch_bounds__(kDecodeThreads) __attribute__((amdgpu_waves_per_eu(2))) void decode_gqa_kernel(DecodeArgs a) {
  constexpr int D = 128, TC = 4, G = C * TC, CPT = D / C;
  constexpr int CW = G / 8;           // uint4 per codeword (fp16, step-major)
  // Codeword stride in uint4: one pad slot makes it odd, so the step-m slices
  // of random codewords spread over all LDS bank groups.
  constexpr int CWS = CW + 1;
  constexpr int DW = C / 2;           // dwords of one step of a codeword
  constexpr int SOFF = 2 * C;         // bytes of one step of a codeword
  constexpr int RW = CPT / 16;        // uint4 per index row
  constexpr int NW = kDecodeThreads / kWave;
  constexpr int TILE = 16;            // tokens per score tile; two tiles per wave iteration
  constexpr int SROW = D + 8;         // fp16 per staged bf16 value row
  // K and V codebooks; after the quantized tokens the same memory holds the
  // staged bf16 values, then the per-wave partial rows of the final merge.
  constexpr int KV_U4 = 2 * 256 * CWS;
  constexpr int RED_U4 = (NW * 16 * (D + 2) * 4 + 15) / 16;
  constexpr int STG_U4 = NW * TILE * SROW * 2 / 16;
  constexpr int U4a = KV_U4 > RED_U4 ? KV_U4 : RED_U4;
  constexpr int U4 = U4a > STG_U4 ? U4a : STG_U4;
  __shared__ __attribute__((aligned(16))) uint4 s_kv[U4];
  uint4* const s_k = s_kv;
  uint4* const s_v = s_kv + 256 * CWS;
  float (*const s_red)[16][D + 2] = reinterpret_cast<float (*)[16][D + 2]>(s_kv);
  uint16_t (*const s_stage)[TILE][SROW] = reinterpret_cast<uint16_t (*)[TILE][SROW]>(s_kv);
  __shared__ float s_amax[3][NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t16 = lane & 15, q4 = lane >> 4;     // key role: token, channel quarter
  const int rho = lane & 15, grp = lane >> 4;    // row role: row (head rho/4, step rho%4), token group
  const int mrow = rho & 3;                      // the row's step within the block
  const int va = lane & 3, vj = (lane >> 2) & 3; // V request role: channel quad, token within the group
  const int split = blockIdx.x;
  const int hq0 = blockIdx.y * HPW;
  const int h = hq0 / a.gqa;
  const int b = blockIdx.z / a.n_blk_serv;
  const int beta = a.blk0 + (blockIdx.z - b * a.n_blk_serv);
  const int t_lo = max(a.step0, beta * TC), t_hi = min(a.step0 + a.n_steps, (beta + 1) * TC);
  // ONE: a single served step m0 of the block; only its codeword slices are
  // read and rotated, and only its rows carry queries
  constexpr int NS = ONE ? 1 : TC;
  const int m0 = ONE ? a.step0 - beta * TC : 0;

  // ---- codebooks -> LDS (fp16, step-major), power-of-two range scaling
  const int64_t cbo = ((int64_t)h * a.n_blk + beta) * a.K * G;
  const int r = tid;
  float kx[G], vx[G];
  float mq, mk, mv;   // the bf16 sinks and recent rows share the codebooks' scales
  decode_input_absmax(a, b, hq0, HPW, h, t_lo, t_hi, split == 0, nullptr, mq, mk, mv);
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
  const int shk = pow2_range_shift(mk, 14), shv = pow2_range_shift(mv, kGVLim), shq = pow2_range_shift(mq, 14);
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

  // ---- query operand (B of the score product): column rho = lane % 16,
  // k quarter kq = lane / 16; block r' holds channels 32r' + 8kq .. +7.
  h8_t qa[4];
  {
    const float qsc = ldexpf(1.f, -shq);
    const int hh = rho >> 2, m = rho & 3, kq = lane >> 4;
    const int t = beta * TC + m;
    const bool act = hh < HPW && t >= t_lo && t < t_hi;
    const uint16_t* qr = a.q + (((int64_t)b * a.Hq + hq0 + (act ? hh : 0)) * a.n_steps + (act ? t - a.step0 : 0)) * D;
#pragma unroll
    for (int rp = 0; rp < 4; ++rp) {
      const uint4 w = *reinterpret_cast<const uint4*>(qr + 32 * rp + 8 * kq);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qa[rp][2 * e] = act ? (_Float16)(bf16lo(ws[e]) * qsc) : (_Float16)0.f;
        qa[rp][2 * e + 1] = act ? (_Float16)(bf16hi(ws[e]) * qsc) : (_Float16)0.f;
      }
    }
  }
  const float sscale = a.qscale * ldexpf(1.f, shk + shq);

  // row-role state: online softmax of row rho and O^T[16b + 4grp + e][rho]
  float Mr = -INFINITY, Lr = 0.f;
  f4g_t oacc[8];
#pragma unroll
  for (int bl = 0; bl < 8; ++bl) oacc[bl] = (f4g_t){0.f, 0.f, 0.f, 0.f};
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

  // Scores of one 16-token tile.  Key lane data: Kc[m][r'] = 8 channels
  // 32r' + 8q4 .. +7 of step m as four fp16 pairs (before rotation); cos/sin:
  // quads 8r + 2q4 and 8r + 2q4 + 1 for r in {0, 1}.  Chain m holds
  // S^T[token][rho] of every row against the keys of step m; row lanes keep
  // the chain of their own step: s[e] = score of row rho, token 4grp + e.
  auto score_tile = [&](uint32_t (&Kc)[NS][4][4], const uint4 (&CS)[2][2], float (&s)[4]) {
    f4g_t ch[NS];
#pragma unroll
    for (int m = 0; m < NS; ++m) ch[m] = (f4g_t){0.f, 0.f, 0.f, 0.f};
    // the four chains interleave, so no MFMA waits for its predecessor
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      h8_t b1[NS], b2[NS];
#pragma unroll
      for (int m = 0; m < NS; ++m) {
        uint32_t o1[4], o2[4];
#pragma unroll
        for (int ip = 0; ip < 4; ++ip) {
          const uint4 q = CS[rr][ip >> 1];
          const h2g_t c2 = as_h2g((ip & 1) ? q.y : q.x), s2 = as_h2g((ip & 1) ? q.w : q.z);
          const h2g_t x1 = as_h2g(Kc[m][rr][ip]), x2 = as_h2g(Kc[m][rr + 2][ip]);
          o1[ip] = __builtin_bit_cast(uint32_t, x1 * c2 - x2 * s2);
          o2[ip] = __builtin_bit_cast(uint32_t, x2 * c2 + x1 * s2);
        }
        b1[m] = __builtin_bit_cast(h8_t, make_uint4(o1[0], o1[1], o1[2], o1[3]));
        b2[m] = __builtin_bit_cast(h8_t, make_uint4(o2[0], o2[1], o2[2], o2[3]));
      }
#pragma unroll
      for (int m = 0; m < NS; ++m) ch[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b1[m], qa[rr], ch[m], 0, 0, 0);
#pragma unroll
      for (int m = 0; m < NS; ++m) ch[m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b2[m], qa[rr + 2], ch[m], 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if constexpr (ONE) {
        s[e] = ch[0][e];
      } else {
        const float v01 = (mrow & 1) ? ch[1][e] : ch[0][e];
        const float v23 = (mrow & 1) ? ch[NS - 1][e] : ch[NS - 2][e];
        s[e] = (mrow & 2) ? v23 : v01;
      }
    }
  };

  // Online softmax of row rho over eight scores (invalid ones already
  // -inf); returns the P operand (fp16, rounded toward zero; the row sum adds
  // the same rounded values).
  auto softmax_rows = [&](float (&s)[8]) {
    float mx = s[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) mx = fmaxf(mx, s[k]);
    mx = group4_max(mx);
    float alpha = 1.f;
    bool moved = false;
    if (mx > Mr + (float)kGLag) {
      alpha = Mr == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mr - mx);
      Mr = mx;
      Lr *= alpha;
      moved = true;
    }
    if (__builtin_expect(__ballot(moved) != 0, 0)) {
#pragma unroll
      for (int bl = 0; bl < 8; ++bl) oacc[bl] *= alpha;
    }
    uint32_t pk[4];
    const h2g_t ones = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float p0 = Mr == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[2 * k] - Mr);
      const float p1 = Mr == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s[2 * k + 1] - Mr);
      const h2g_t ph = __builtin_bit_cast(h2g_t, __builtin_amdgcn_cvt_pkrtz(p0, p1));
      Lr = __builtin_amdgcn_fdot2(ph, ones, Lr, false);
      pk[k] = __builtin_bit_cast(uint32_t, ph);
    }
    return __builtin_bit_cast(h8_t, make_uint4(pk[0], pk[1], pk[2], pk[3]));
  };
  auto load_cs = [&](int pos, uint4 (&CS)[2][2]) {
    const uint4* row = reinterpret_cast<const uint4*>(rope16 + (int64_t)pos * D);
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int u = 0; u < 2; ++u) CS[rr][u] = row[8 * rr + 2 * q4 + u];
  };

  // ---- quantized tokens: 32 per wave iteration (two score tiles), index
  // rows of the next iteration loaded while this one is computed
  const int n_tok = max(0, tok_hi - tok_lo);
  uint4 krow[2][RW], vrow[2][RW];
  auto load_rows = [&](int base, uint4 (&kr)[2][RW], uint4 (&vr)[2][RW]) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int ik = base + wave * 2 * TILE + TILE * hf + t16;
      const int iv = base + wave * 2 * TILE + TILE * hf + 4 * grp + vj;
      const int64_t jk = tok_lo + (ik < n_tok ? ik : n_tok - 1);   // always a real row
      const int64_t jv = tok_lo + (iv < n_tok ? iv : n_tok - 1);
      const uint4* pk = reinterpret_cast<const uint4*>(a.kidx + (irow0 + jk) * CPT);
      const uint4* pv = reinterpret_cast<const uint4*>(a.vidx + (irow0 + jv) * CPT);
#pragma unroll
      for (int u = 0; u < RW; ++u) {
        kr[hf][u] = pk[u];
        vr[hf][u] = pv[u];
      }
    }
  };
  // K codewords of the chunks holding channels 32r + 8q4 + j (j < 8)
  auto gather_k = [&](const uint4 (&kr)[RW], uint32_t (&Kc)[NS][4][4]) {
    uint32_t kd[4 * RW];
#pragma unroll
    for (int u = 0; u < RW; ++u) {
      kd[4 * u] = kr[u].x; kd[4 * u + 1] = kr[u].y; kd[4 * u + 2] = kr[u].z; kd[4 * u + 3] = kr[u].w;
    }
#pragma unroll
    for (int rp = 0; rp < 4; ++rp) {
      if constexpr (C == 8) {
        const int c = 4 * rp + q4;                          // chunk = channels 8c .. 8c+7
        const uint32_t ik = __builtin_amdgcn_ubfe(kd[c >> 2], 8 * (c & 3), 8);
        const uint4* cw = &s_k[ik * CWS];
#pragma unroll
        for (int m = 0; m < NS; ++m) {
          const uint4 x = cw[ONE ? m0 : m];                 // step m: 8 channels
          Kc[m][rp][0] = x.x; Kc[m][rp][1] = x.y; Kc[m][rp][2] = x.z; Kc[m][rp][3] = x.w;
        }
      } else {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int c = 8 * rp + 2 * q4 + half;             // chunk = channels 4c .. 4c+3
          const uint32_t ik = __builtin_amdgcn_ubfe(kd[c >> 2], 8 * (c & 3), 8);
          const uint4* cw = &s_k[ik * CWS];
          if constexpr (ONE) {
            const uint2 x = reinterpret_cast<const uint2*>(cw)[m0];   // step m0: 4 channels
            Kc[0][rp][2 * half] = x.x; Kc[0][rp][2 * half + 1] = x.y;
          } else {
            const uint4 x0 = cw[0], x1 = cw[1];             // steps 0-1, 2-3
            Kc[0][rp][2 * half] = x0.x; Kc[0][rp][2 * half + 1] = x0.y;
            Kc[1][rp][2 * half] = x0.z; Kc[1][rp][2 * half + 1] = x0.w;
            Kc[NS - 2][rp][2 * half] = x1.x; Kc[NS - 2][rp][2 * half + 1] = x1.y;
            Kc[NS - 1][rp][2 * half] = x1.z; Kc[NS - 1][rp][2 * half + 1] = x1.w;
          }
        }
      }
    }
  };
  // LDS byte offset (from s_v) of this request lane's step-0 slice of the V
  // codeword of chunk block bl, token of the given index row: channels
  // 16bl + 4va .. +3.
  auto v_off = [&](const uint4 (&vr)[RW], int bl) -> uint32_t {
    uint32_t vd[4 * RW];
#pragma unroll
    for (int u = 0; u < RW; ++u) {
      vd[4 * u] = vr[u].x; vd[4 * u + 1] = vr[u].y; vd[4 * u + 2] = vr[u].z; vd[4 * u + 3] = vr[u].w;
    }
    if constexpr (C == 8) {
      // chunk 2bl + va/2, byte 2(bl & 1) + va/2 of dword bl/2; half va & 1 of the step slice
      const uint32_t ix = __builtin_amdgcn_ubfe(vd[bl >> 1], 16 * (bl & 1) + 8 * (va >> 1), 8);
      return ix * (CWS * 16) + 8 * (va & 1);
    } else {
      // chunk 4bl + va: byte va of dword bl
      const uint32_t ix = __builtin_amdgcn_ubfe(vd[bl], 8 * va, 8);
      return ix * (CWS * 16);
    }
  };

  uint4 CS[2][2];
  if (n_tok > 0) {
    load_rows(0, krow, vrow);
    load_cs(a.n_s + tok_lo + min(wave * 2 * TILE + t16, n_tok - 1), CS);
  }
  for (int base = 0; base < n_tok; base += NW * 2 * TILE) {
    const int w0 = base + wave * 2 * TILE;
    float s[8];
    {
      uint32_t Kc[NS][4][4];
      gather_k(krow[0], Kc);
      float s0[4];
      score_tile(Kc, CS, s0);
      load_cs(a.n_s + tok_lo + min(w0 + TILE + t16, n_tok - 1), CS);
      gather_k(krow[1], Kc);
      float s1[4];
      score_tile(Kc, CS, s1);
      load_cs(a.n_s + tok_lo + min(w0 + NW * 2 * TILE + t16, n_tok - 1), CS);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[e] = w0 + 4 * grp + e < n_tok ? s0[e] * sscale : -INFINITY;
        s[4 + e] = w0 + TILE + 4 * grp + e < n_tok ? s1[e] * sscale : -INFINITY;
      }
    }
    const h8_t P = softmax_rows(s);
    uint32_t voff[2][8];
#pragma unroll
    for (int bl = 0; bl < 8; ++bl) {
      voff[0][bl] = v_off(vrow[0], bl);
      voff[1][bl] = v_off(vrow[1], bl);
    }
    if (base + NW * 2 * TILE < n_tok) load_rows(base + NW * 2 * TILE, krow, vrow);
#pragma unroll
    for (int mi = 0; mi < NS; ++mi) {
      const int m = ONE ? m0 : mi;
      const h8_t Pm = ONE || mrow == m ? P : (h8_t){};
#pragma unroll
      for (int bl = 0; bl < 8; ++bl) {
        const h4g_t lo = lds_tr4(s_v, voff[0][bl] + SOFF * m);
        const h4g_t hi = lds_tr4(s_v, voff[1][bl] + SOFF * m);
        const h8_t A = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[bl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Pm, oacc[bl], 0, 0, 0);
      }
    }
  }

  // ---- bf16 items (split 0): sinks at positions 0..n_s-1, then the recent
  // window at n_s + N_b + r; 16 per wave iteration, their values staged per
  // step in this wave's LDS rows (the codebook memory, once every wave is done
  // with it)
  __syncthreads();
  for (int base = 0; base < n_bf; base += NW * TILE) {
    const int w0 = base + wave * TILE;
    float s[8];
    {
      const int item = w0 + t16;
      const int it = item < n_bf ? item : 0;
      const bool is_rec = it >= n_sink;
      const int pos = is_rec ? a.n_s + nb + (it - n_sink) : it;
      uint32_t Kc[NS][4][4];
#pragma unroll
      for (int mi = 0; mi < NS; ++mi) {
        const int m = ONE ? m0 : mi;
        const uint16_t* kr = is_rec ? a.rk + (rec0 + (int64_t)m * a.r_cap + (it - n_sink)) * D
                                    : a.sk + (sink0 + (int64_t)m * a.n_s + it) * D;
#pragma unroll
        for (int rp = 0; rp < 4; ++rp) {
          const uint4 w = *reinterpret_cast<const uint4*>(kr + 32 * rp + 8 * q4);
          const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) Kc[mi][rp][e] = pack_h2g(bf16lo(ws[e]) * ksc, bf16hi(ws[e]) * ksc);
        }
      }
      uint4 CSb[2][2];
      load_cs(pos, CSb);
      float s0[4];
      score_tile(Kc, CSb, s0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s[e] = w0 + 4 * grp + e < n_bf ? s0[e] * sscale : -INFINITY;
        s[4 + e] = -INFINITY;
      }
    }
    const h8_t P = softmax_rows(s);
    // staging lane: item w0 + lane/4, channels 32 (lane & 3) .. +31
    const int si = lane >> 2, sc = 32 * (lane & 3);
    const int sit = w0 + si < n_bf ? w0 + si : 0;
    const bool s_rec = sit >= n_sink;
#pragma unroll 1
    for (int mi = 0; mi < NS; ++mi) {
      const int m = ONE ? m0 : mi;
      const uint16_t* vr = s_rec ? a.rv + (rec0 + (int64_t)m * a.r_cap + (sit - n_sink)) * D
                                 : a.sv + (sink0 + (int64_t)m * a.n_s + sit) * D;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 w = *reinterpret_cast<const uint4*>(vr + sc + 8 * u);
        *reinterpret_cast<uint4*>(&s_stage[wave][si][sc + 8 * u]) =
            make_uint4(pack_h2g(bf16lo(w.x) * vsc, bf16hi(w.x) * vsc), pack_h2g(bf16lo(w.y) * vsc, bf16hi(w.y) * vsc),
                       pack_h2g(bf16lo(w.z) * vsc, bf16hi(w.z) * vsc), pack_h2g(bf16lo(w.w) * vsc, bf16hi(w.w) * vsc));
      }
      wave_sync();
      const h8_t Pm = ONE || mrow == m ? P : (h8_t){};
      const uint32_t roff = (uint32_t)((4 * grp + vj) * SROW + 4 * va) * 2;
#pragma unroll
      for (int bl = 0; bl < 8; ++bl) {
        const h4g_t lo = lds_tr4(&s_stage[wave][0][0], roff + 32 * bl);
        const h8_t A = __builtin_shufflevector(lo, (h4g_t){}, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[bl] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Pm, oacc[bl], 0, 0, 0);
      }
      wave_sync();
    }
  }

  // ---- per-wave row totals, then merge the waves through LDS
  __syncthreads();
  {
    const float l = group4_sum(Lr);
    if (grp == 0) {
      s_red[wave][rho][D] = Mr;
      s_red[wave][rho][D + 1] = l;
    }
  }
#pragma unroll
  for (int bl = 0; bl < 8; ++bl)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_red[wave][rho][16 * bl + 4 * grp + e] = oacc[bl][e];
  __syncthreads();
  const float osc = ldexpf(1.f, shv);
  for (int x = tid; x < 16 * D; x += kDecodeThreads) {
    const int rw = x / D, d = x - rw * D;
    const int hh = rw >> 2, m = rw & 3;
    const int t = beta * TC + m;
    if (hh >= HPW || t < t_lo || t >= t_hi) continue;
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, s_red[w][rw][D]);
    float num = 0.f, den = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = s_red[w][rw][D];
        const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mm);
        num += f * s_red[w][rw][d];
        den += f * s_red[w][rw][D + 1];
      }
    }
    const int64_t row = ((int64_t)b * a.Hq + hq0 + hh) * a.n_steps + (t - a.step0);
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

template <int C, bool ONE>
static hipError_t launch_gqa_c(int hpw, const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.n_split, a.Hq / hpw, a.B * a.n_blk_serv);
  if (hpw == 4)
    hipLaunchKernelGGL((decode_gqa_kernel<C, 4, ONE>), grid, dim3(kDecodeThreads), 0, s, a);
  else if (hpw == 2)
    hipLaunchKernelGGL((decode_gqa_kernel<C, 2, ONE>), grid, dim3(kDecodeThreads), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_gqa(int G, int hpw, const DecodeArgs& a, hipStream_t s) {
  // one served step: only that step's slices are read (the plan serves it in
  // a single block)
  const bool one = a.n_steps == 1;
  if (G == 16) return one ? launch_gqa_c<4, true>(hpw, a, s) : launch_gqa_c<4, false>(hpw, a, s);
  if (G == 32) return one ? launch_gqa_c<8, true>(hpw, a, s) : launch_gqa_c<8, false>(hpw, a, s);
  return hipErrorInvalidValue;
}

}  // namespace loopvq
