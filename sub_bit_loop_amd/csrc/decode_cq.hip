// LoopVQ decode attention over per-step codebooks (T_c = 1, G = 16: one
// 8-bit code covers 16 channels of one loop step, 0.5 bit per element), no
// channel pre-transform.
//
// LoopVQ review (arXiv 2611.05304), section 2 eq. (2) (plain channel VQ: a
// code covers G consecutive channels of one step) and section 3.3 (per-step
// codebooks for the layers outside the loop); section 3.4 step 3 (codebook on
// chip, lookup by index, RoPE from a precomputed table after dequant,
// Flash-Decoding split merge).
//
// With T_c = 1 every block is one step with its own codebook, so a workgroup
// serves one (batch, q-head, step, context split) and all four waves take
// different tokens of that step:
//   * A token is served by four lanes of a wave (16 tokens per wave).  Lane g
//     owns chunk g (channels 16g .. 16g+15) and its RoPE partner chunk g + 4
//     (channels 64+16g ..): bytes g of the two index dwords.
//   * Codewords sit in LDS as fp16 (16 channels, 32 bytes) with a stride of
//     three 16-byte slots; codebooks are rescaled by powers of two on load
//     (keys to fit fp16, values below 2^kCVLim; the bf16 sinks and recent
//     rows count in those ranges) and the queries by one of their own; the
//     scales are folded back later.
//   * Rotation on packed fp16 pairs, scores as v_dot2_f32_f16 sums, the four
//     lanes of a token reduce with DPP, online softmax in base 2 whose running
//     maximum may lag by kCLag, and P*V in packed fp16 flushed into fp32 every
//     kCFlush tokens.
#include "common.h"
#include "kernels.h"

namespace loopvq {

namespace {

typedef _Float16 hc2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ hc2_t as_hc2(uint32_t w) { return __builtin_bit_cast(hc2_t, w); }

__device__ __forceinline__ uint32_t pack_hc2(float a, float b) {
  const _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// fp16 partial sums of P*V: weights <= 2^kCLag, |v| <= 2^kCVLim, kCFlush tokens
// per lane between flushes keep a partial below 2^(3+7+4) = 16384.
constexpr int kCFlush = 16, kCLag = 3, kCVLim = 7;
constexpr int kCQS = 3;                 // LDS slots of 16 bytes per codeword (2 used)

}  // namespace

__global__ __launch_bounds__(kDecodeThreads) void decode_cq_kernel(DecodeArgs a) {
  constexpr int D = 128, HD = 64, G = 16, CPT = D / G, NW = kDecodeThreads / kWave, SPW = 16;
  __shared__ __attribute__((aligned(16))) uint4 s_k[256 * kCQS];
  __shared__ __attribute__((aligned(16))) uint4 s_v[256 * kCQS];
  __shared__ float s_red[NW][D + 2];
  __shared__ float s_amax[3][NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = lane >> 2, g = lane & 3;
  const int split = blockIdx.x;
  const int hq = blockIdx.y;
  const int h = hq / a.gqa;
  const int b = blockIdx.z / a.n_blk_serv;
  const int beta = a.blk0 + (blockIdx.z - b * a.n_blk_serv);   // block = step
  const bool served = beta >= a.step0 && beta < a.step0 + a.n_steps;

  // ---- codebooks -> LDS (fp16), power-of-two range scaling
  const int64_t cbo = ((int64_t)h * a.n_blk + beta) * a.K * G;
  int shk, shv, shq;
  {
    const int r = tid;   // one row per thread
    float kx[G], vx[G];
    float mq, mk, mv;   // the bf16 sinks and recent rows share the codebooks' scales
    if (served)
      decode_input_absmax(a, b, hq, 1, h, beta, beta + 1, split == 0, nullptr, mq, mk, mv);
    else
      mq = mk = mv = 0.f;
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
    shq = pow2_range_shift(mq, 14);
    shk = pow2_range_shift(mk, 14);
    shv = pow2_range_shift(mv, kCVLim);
    const float sk = ldexpf(1.f, -shk), sv = ldexpf(1.f, -shv);
    uint32_t kw[8], vw[8];
#pragma unroll
    for (int ip = 0; ip < 8; ++ip) {
      kw[ip] = pack_hc2(kx[2 * ip] * sk, kx[2 * ip + 1] * sk);
      vw[ip] = pack_hc2(vx[2 * ip] * sv, vx[2 * ip + 1] * sv);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s_k[r * kCQS + u] = make_uint4(kw[4 * u], kw[4 * u + 1], kw[4 * u + 2], kw[4 * u + 3]);
      s_v[r * kCQS + u] = make_uint4(vw[4 * u], vw[4 * u + 1], vw[4 * u + 2], vw[4 * u + 3]);
    }
  }
  __syncthreads();

  // query of this step: chunk g (channel pairs 16g + 2i) and its partner chunk
  const uint16_t* qr = a.q + (((int64_t)b * a.Hq + hq) * a.n_steps + (served ? beta - a.step0 : 0)) * D;
  uint32_t q1[8], q2[8];
  const float qsc = ldexpf(1.f, -shq);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w1 = *reinterpret_cast<const uint32_t*>(qr + 16 * g + 2 * i);
    const uint32_t w2 = *reinterpret_cast<const uint32_t*>(qr + HD + 16 * g + 2 * i);
    q1[i] = served ? pack_hc2(bf16lo(w1) * qsc, bf16hi(w1) * qsc) : 0u;
    q2[i] = served ? pack_hc2(bf16lo(w2) * qsc, bf16hi(w2) * qsc) : 0u;
  }
  const float sscale = a.qscale * ldexpf(1.f, shk + shq);

  float mrow = -INFINITY, lrow = 0.f;
  float acc[2][16];
  uint32_t acc16[2][8];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[p][c] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc16[p][i] = 0u;
  }

  int nb = a.N;
  if (a.seq_len) nb = max(0, min(a.seq_len[b], a.N));
  const int tok_lo = split * a.tok_per_split;
  const int tok_hi = min(nb, tok_lo + a.tok_per_split);
  const int n_sink = split == 0 ? a.n_s : 0;
  const int n_bf = n_sink + (split == 0 ? a.n_r : 0);
  const int64_t irow0 = (((int64_t)b * a.H + h) * a.n_blk + beta) * (int64_t)a.N_cap;
  const int64_t sink0 = (((int64_t)b * a.H + h) * a.T + beta) * (int64_t)a.n_s;
  const int64_t rec0 = (((int64_t)b * a.H + h) * a.T + beta) * (int64_t)a.r_cap;
  const uint16_t* rope16 = reinterpret_cast<const uint16_t*>(a.rope);
  const float ksc = ldexpf(1.f, -shk), vsc = ldexpf(1.f, -shv);

  // Kw[p][i]: channel pair i of chunk g (p = 0) or of its partner (p = 1);
  // CS[k]: cos/sin quad of frequencies 16g + 4k .. +3.
  auto score = [&](const uint32_t (&Kw)[2][8], const uint4 (&CS)[4]) {
    float sc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 q4 = CS[i >> 1];
      const hc2_t c2 = as_hc2((i & 1) ? q4.y : q4.x), s2 = as_hc2((i & 1) ? q4.w : q4.z);
      const hc2_t x1 = as_hc2(Kw[0][i]), x2 = as_hc2(Kw[1][i]);
      const hc2_t r1 = x1 * c2 - x2 * s2;
      const hc2_t r2 = x2 * c2 + x1 * s2;
      sc = __builtin_amdgcn_fdot2(r1, as_hc2(q1[i]), sc, false);
      sc = __builtin_amdgcn_fdot2(r2, as_hc2(q2[i]), sc, false);
    }
    return group_sum<4>(sc) * sscale;
  };
  auto flush = [&]() {
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        add_f16x2(acc16[p][i], acc[p][2 * i], acc[p][2 * i + 1]);
        acc16[p][i] = 0u;
      }
  };
  auto accumulate = [&](float s, const uint32_t (&Vw)[2][8], bool valid) {
    if (!valid) return;
    if (s > mrow + (float)kCLag) {
      const float alpha = __builtin_amdgcn_exp2f(mrow - s);
      const hc2_t a2 = {(_Float16)alpha, (_Float16)alpha};
      lrow *= alpha;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int c = 0; c < 16; ++c) acc[p][c] *= alpha;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc16[p][i] = __builtin_bit_cast(uint32_t, as_hc2(acc16[p][i]) * a2);
      }
      mrow = s;
    }
    const float pr = __builtin_amdgcn_exp2f(s - mrow);
    lrow += pr;
    const hc2_t p2 = {(_Float16)pr, (_Float16)pr};
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc16[p][i] = __builtin_bit_cast(uint32_t, as_hc2(Vw[p][i]) * p2 + as_hc2(acc16[p][i]));
  };
  auto load_cs = [&](int pos, uint4 (&CS)[4]) {
    const uint4* row = reinterpret_cast<const uint4*>(rope16 + (int64_t)pos * D);
#pragma unroll
    for (int k = 0; k < 4; ++k) CS[k] = row[4 * g + k];
  };
  auto gather = [&](const uint4* cb, uint32_t ix, uint32_t (&out)[8]) {
    const uint4 x = cb[ix * kCQS], y = cb[ix * kCQS + 1];
    out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
    out[4] = y.x; out[5] = y.y; out[6] = y.z; out[7] = y.w;
  };

  // Sinks and the recent window (split 0 only), straight from the bf16 rows,
  // scaled like the codebooks.  Sink s sits at position s, recent token r at
  // n_s + N_b + r.
  if (served) {
    for (int base = 0; base < n_bf; base += NW * SPW) {
      const int item = base + wave * SPW + slot;
      const bool valid = item < n_bf;
      const int it = valid ? item : 0;
      const bool is_rec = it >= n_sink;
      const int pos = is_rec ? a.n_s + nb + (it - n_sink) : it;
      const uint16_t* kr = is_rec ? a.rk + (rec0 + (it - n_sink)) * D : a.sk + (sink0 + it) * D;
      const uint16_t* vr = is_rec ? a.rv + (rec0 + (it - n_sink)) * D : a.sv + (sink0 + it) * D;
      uint32_t Kw[2][8], Vw[2][8];
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t x = *reinterpret_cast<const uint32_t*>(kr + p * HD + 16 * g + 2 * i);
          const uint32_t y = *reinterpret_cast<const uint32_t*>(vr + p * HD + 16 * g + 2 * i);
          Kw[p][i] = pack_hc2(bf16lo(x) * ksc, bf16hi(x) * ksc);
          Vw[p][i] = pack_hc2(bf16lo(y) * vsc, bf16hi(y) * vsc);
        }
      uint4 CS[4];
      load_cs(pos, CS);
      accumulate(score(Kw, CS), Vw, valid);
      flush();
    }
  }

  // Context tokens: the two index dwords of a row, loaded one iteration ahead
  // with the sin/cos quads.
  const int n_tok = served ? max(0, tok_hi - tok_lo) : 0;
  const int my = wave * SPW + slot;
  uint2 kd, vd;
  uint4 CS[4];
  auto load_rows = [&](int base, int& jj) {
    const int it = base + my;
    jj = tok_lo + (it < n_tok ? it : n_tok - 1);   // always a real row
    kd = *reinterpret_cast<const uint2*>(a.kidx + (irow0 + jj) * CPT);
    vd = *reinterpret_cast<const uint2*>(a.vidx + (irow0 + jj) * CPT);
  };
  if (n_tok > 0) {
    int jj;
    load_rows(0, jj);
    load_cs(a.n_s + jj, CS);
  }
  int since_flush = 0;
  for (int base = 0; base < n_tok; base += NW * SPW) {
    const bool valid = base + my < n_tok;
    const uint32_t ka0 = __builtin_amdgcn_ubfe(kd.x, 8 * g, 8), ka1 = __builtin_amdgcn_ubfe(kd.y, 8 * g, 8);
    const uint32_t va0 = __builtin_amdgcn_ubfe(vd.x, 8 * g, 8), va1 = __builtin_amdgcn_ubfe(vd.y, 8 * g, 8);
    int jn;
    load_rows(base + NW * SPW, jn);
    uint32_t Kw[2][8], Vw[2][8];
    gather(s_k, ka0, Kw[0]);
    gather(s_k, ka1, Kw[1]);
    gather(s_v, va0, Vw[0]);
    gather(s_v, va1, Vw[1]);
    const float s = score(Kw, CS);
    load_cs(a.n_s + jn, CS);
    accumulate(s, Vw, valid);
    if (++since_flush == kCFlush) {
      flush();
      since_flush = 0;
    }
  }
  flush();

  // merge the 16 token slots of the wave (lanes with equal g), then the waves
#pragma unroll
  for (int off = 4; off < kWave; off <<= 1) {
    const float om = __shfl_xor(mrow, off);
    const float ol = __shfl_xor(lrow, off);
    const float mm = fmaxf(mrow, om);
    const float a1 = mrow == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrow - mm);
    const float a2 = om == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(om - mm);
    lrow = lrow * a1 + ol * a2;
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float oa = __shfl_xor(acc[p][c], off);
        acc[p][c] = acc[p][c] * a1 + oa * a2;
      }
    mrow = mm;
  }
  if (slot == 0) {
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int c = 0; c < 16; ++c) s_red[wave][p * HD + 16 * g + c] = acc[p][c];
    if (g == 0) {
      s_red[wave][D] = mrow;
      s_red[wave][D + 1] = lrow;
    }
  }
  __syncthreads();
  if (!served) return;
  const float osc = ldexpf(1.f, shv);
  for (int d = tid; d < D; d += kDecodeThreads) {
    float mm = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, s_red[w][D]);
    float num = 0.f, den = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = s_red[w][D];
        const float f = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - mm);
        num += f * s_red[w][d];
        den += f * s_red[w][D + 1];
      }
    }
    float* dst = a.ws + ((((int64_t)b * a.Hq + hq) * a.n_steps + (beta - a.step0)) * a.n_split + split) * (D + 1);
    dst[d] = den > 0.f ? num / den * osc : 0.f;
    if (d == 0) dst[D] = den > 0.f ? (mm + __log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
}

hipError_t launch_decode_cq(const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.Hq, a.B * a.n_blk_serv);
  hipLaunchKernelGGL(decode_cq_kernel, grid, dim3(kDecodeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace loopvq
