// LoopVQ fused decode attention for keys stored with the channel
// pre-transform (TaSQ), blocks of T_c = 4 loop steps, c = 4 or 8 channels per
// step per code, D = 128.
//
// LoopVQ review (arXiv 2611.05304), section 3.3 eq. (10) (keys multiplied by
// per-channel weights, divided by the token's scale sigma and permuted before
// grouping; the inverse is applied at dequant), section 3.4 step 3 (codebook
// on chip, lookup by index, RoPE from a precomputed table after dequant,
// Flash-Decoding split merge) and section 3.1 eq. (5) (step m reads
// coordinate i*T_c + m of the shared codeword).
//
// The restored key is k[p(d')] = sigma * z[d'] / w[p(d')] (p = permutation,
// z = codeword slice in the transformed space), rotated by RoPE at the token
// position.  Since q . R_pos k = (R_-pos q) . k, a key is scored in the
// transformed space against an effective query
//     e[d'] = a[d'] cos(pos w_f) + b[d'] sin(pos w_f),   f = p(d') mod D/2,
//     a[d'] = q[p(d')] / w[p(d')],
//     b[d'] = +-q[p(d') +- D/2] / w[p(d')]   (+ for p(d') < D/2),
// and the dot product is multiplied by the token's sigma.  The permutation
// separates RoPE partners, so unlike the plain kernels no lane rotates a key.
//
// Positions: a workgroup iteration serves 4 consecutive tokens per wave (8
// with one served step) at positions P + o, where P is the same for every
// lane and o is fixed per lane.  The waves run their iterations without
// waiting for each other; the issue arbitration favours older waves, so every
// 16 iterations a wave that has done fewer than the workgroup's average
// raises its priority (s_setprio) until it catches up, and the waves finish
// together (each token still goes to the same lane in the same order).
// By the angle-sum identity
//     e[d'](P + o) = A_o[d'] cos(P w_f) + B_o[d'] sin(P w_f),
//     A_o = a cos(o w_f) + b sin(o w_f),   B_o = b cos(o w_f) - a sin(o w_f),
// so the per-lane coefficients A_o, B_o are formed once (fp32 angles of
// o w_f).  A lane's 16 transformed channels form 8 channel pairs, and the 8
// lane groups of a token hold 64 pairs in all, so per iteration lane
// 8p + g of each wave loads the table entries (cos P w_f, sin P w_f) of the
// two frequencies of pair p of group g and stores them as one 8-byte entry
// (cos pair, sin pair) of the wave's LDS table; every lane then reads its 8
// pairs' entries, already packed for the fp16 pair arithmetic.  Both the
// store and each read cover consecutive entries, so neither meets a bank
// conflict (lanes reading one entry share it).
//
// Layout choices:
//   * Codebooks in LDS as fp16, step-major inside a codeword, first half
//     steps 0-1, second half steps 2-3 (as in the plain multi-step kernel).
//     With c = 4 and every step served, eight copies, one per lane group, so
//     that the gathers meet no bank conflicts (a workgroup of 12 waves then
//     fills a CU's LDS).
//   * 16 lanes serve a token: lane (hs, g) takes steps {2hs, 2hs+1} and the
//     chunks D/c/8 * g .. +D/c/8-1, i.e. the 16 transformed channels
//     16g .. 16g+15, whose index bytes are one aligned 4-byte word (c = 4) or
//     half of one (c = 8).
//   * Effective queries, scores and P*V run on packed fp16 (scores summed in
//     fp32 by v_dot2_f32_f16); P*V partials are flushed into fp32 every
//     kTFlush(NSL) tokens, with the same kind of range bounds as the plain kernels.
//   * Online softmax (all steps, NSL = 2): the four tokens of a wave
//     iteration share one running maximum per step, raised in a branch the
//     whole wave takes, so their fp16 partials add up across the four rows
//     before a flush and the wave keeps one set of fp32 sums in LDS; of the
//     two lanes g and 7 - g that hold the same steps, each keeps the softmax
//     of one step and hands its weight to the other through DPP.
// One workgroup serves one (batch, q-head, block, context split).  A call
// for one served step (n_steps = 1) takes the variant with one step per lane
// (NSL = 1): lanes hs = 0 / 1 then serve two tokens instead of two steps, and
// only the served step's slice of each codeword is read.
#include "common.h"
#include "kernels.h"

namespace loopvq {

namespace {

typedef _Float16 h2t_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2t_t as_h2t(uint32_t w) { return __builtin_bit_cast(h2t_t, w); }

// a.x * b.x + a.y * b.y in fp32, the first product of a chain: the VOP3
// form takes the zero addend as a constant (the compiler's accumulating form
// would first move a zero into a register)
__device__ __forceinline__ float dot2_first(h2t_t a, h2t_t b) {
  float r;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// w16 * S + add, w16 the 16-bit half H of w (op_sel picks the high half):
// the byte offset of a codeword from an index spread into a 16-bit half
// (S up to 64 is an inline constant; a larger one sits in a scalar register)
template <int H, int S>
__device__ __forceinline__ uint32_t mad_half(uint32_t w, uint32_t add) {
  uint32_t r;
  if constexpr (S <= 64) {
    if constexpr (H == 0)
      asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(r) : "v"(w), "i"(S), "v"(add));
    else
      asm("v_mad_u32_u16 %0, %1, %2, %3 op_sel:[1,0,0,0]" : "=v"(r) : "v"(w), "i"(S), "v"(add));
  } else {
    if constexpr (H == 0)
      asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(S), "v"(add));
    else
      asm("v_mad_u32_u16 %0, %1, %2, %3 op_sel:[1,0,0,0]" : "=v"(r) : "v"(w), "s"(S), "v"(add));
  }
  return r;
}

__device__ __forceinline__ uint32_t pack_h2t(float a, float b) {
  const _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// P*V partial range: weights below 2^kTLag; a lane's fp16 partial sums at
// most kTFlush(NSL) tokens before it is flushed into fp32, with values below
// 2^kTVLim(NSL), so a partial stays below 2^14, and below 2^15 where four
// rows' partials are added before a flush (NSL = 2: 32 tokens, values below
// 2^5; NSL = 1: 16 tokens, values below 2^7).
constexpr int kTLag = 3;
constexpr int kTFlush(int nsl) { return nsl == 2 ? 32 : 16; }
constexpr int kTVLim(int nsl) { return nsl == 2 ? 5 : 7; }
// Fourth word of a raw buffer descriptor (32-bit data, no format conversion).
constexpr int kBufWord3 = 0x00020000;

}  // namespace

// NSL = 2: every step of the block (lane (hs, g) takes steps 2hs, 2hs+1);
// NSL = 1: one served step (a call with n_steps = 1): lane (hs, g) then takes
// that step for tokens of parity hs, so the 16 lanes of a token pair serve
// two tokens and no lane computes a step that is not served.
template <int C, int NSL>
__global__ __launch_bounds__(tasq_threads(C, NSL), C == 4 ? 1 : (NSL == 1 ? 4 : 2)) void decode_tasq_kernel(
    DecodeArgs a) {
  constexpr int D = 128, HD = 64, TC = 4, G = C * TC, CPT = D / C;
  constexpr int QW = C / 4;           // uint4 per codeword half (two steps)
  constexpr int DW = C / 2;           // dwords per step of a codeword
  // kRep (c = 4, every step): one workgroup of 12 waves per CU, with eight
  // copies of each codebook, one per lane group g: row r (256 bytes) holds
  // codeword r of copy j at bytes 32 j .. 32 j + 31, so the 16 lanes of a
  // token, which read 8 codewords (a half each), meet 8 disjoint sets of
  // banks and a gather has no bank conflict.  The V rows follow the K rows
  // 64 KB further on, so the byte offset of a codeword half, idx * 256 +
  // 32 g + 16 hs (+ 65536 for V), is assembled by one byte permute.
  // kSlice (c = 4, one served step m0): one workgroup of 16 waves per CU,
  // whose LDS holds only step m0's 8-byte slice of each codeword, 16 copies:
  // row r (256 bytes) holds the K slice of copy j at bytes 8 j and the V
  // slice at 128 + 8 j, and lane l reads copy l mod 16, so the 16 lanes of a
  // token pair meet disjoint banks; a slice's offset, idx * 256 + 8 (l mod
  // 16) (+ 128 for V), is again one byte permute.
  // Otherwise (c = 8) one copy of each codebook, codeword r at 32 QW r, and
  // workgroups of 4 waves.
  constexpr int kFl = kTFlush(NSL);
  constexpr bool kRep = C == 4 && NSL == 2;
  constexpr bool kSlice = C == 4 && NSL == 1;
  constexpr int NTH = tasq_threads(C, NSL);
  constexpr int LPT = 16, SPW = kWave / LPT, NW = NTH / kWave;
  constexpr int TPI = NW * SPW * (3 - NSL);   // tokens per workgroup iteration (48, 128, 16 or 32)
  constexpr int NCK = CPT / 8;        // chunks per lane (4 or 2)
  constexpr int NCH = NCK * C;        // transformed channels per lane (16)
  constexpr int NPR = NCH / 2;        // channel pairs per lane (8)
  constexpr int KWD = NSL * DW;       // codeword dwords per chunk a lane reads
  static_assert(NPR * 8 == kWave, "one channel pair of the table per lane");
  constexpr int kRowQ = kRep || kSlice ? 16 : 2 * QW;   // uint4 per codebook row in LDS
  __shared__ __attribute__((aligned(16))) uint4 s_k[256 * kRowQ * (kRep ? 2 : 1)];
  // kRep: the V rows are the second half of s_k; kSlice: the second half of each row
  __shared__ __attribute__((aligned(16))) uint4 s_v[kRep || kSlice ? 1 : 256 * kRowQ];
  uint4* const cbk = s_k;
  uint4* const cbv = kRep ? s_k + 256 * kRowQ : (kSlice ? s_k + 8 : s_v);
  // fp32 P*V sums.  NSL = 2: the four tokens of a wave iteration (lanes l,
  // l ^ 16, l ^ 32, l ^ 48, which hold the same channels and steps) share
  // one running maximum per step, so their fp16 partials add up before a
  // flush and the wave keeps one set of sums, s_red[wave][step][channel],
  // which is also the wave's slot of the final merge.  NSL = 1: every lane
  // keeps its own maximum and sums (quad q of lane t at float4
  // q * 256 + t, which consecutive lanes read without bank conflicts).
  // One region, used in turn for (cos, sin) of o * w_f for o < TPI, f < HD
  // (fp32) while the coefficients are formed, the sums during the token
  // loop, and the cross-wave merge of the partial outputs at the end.
  constexpr bool kShared = NSL == 2;
  constexpr int RW = D + 4;              // merge row: D sums, maximum, sum of weights, padding
  constexpr int kAccQ = NSL * NCH / 4;   // NSL = 1: float4 sums per lane
  constexpr int kRedQ = NW * TC * RW / 4, kOffQ = TPI * HD / 2, kLaneQ = kShared ? 0 : kAccQ * NTH;
  constexpr int kBufQ = kRedQ > kOffQ ? (kRedQ > kLaneQ ? kRedQ : kLaneQ) : (kOffQ > kLaneQ ? kOffQ : kLaneQ);
  __shared__ __attribute__((aligned(16))) float4 s_buf[kBufQ];
  __shared__ float s_amax[3][NW];
  __shared__ int s_prog;   // blocks of kTFlush(NSL) iterations done by the workgroup's waves
  // (cos, sin) of the iteration's position for every channel pair: entry
  // 8p + g holds pair p of lane group g, as (cos of both, sin of both) fp16
  __shared__ uint2 s_pair[NW][NPR * 8];
  float (*s_red)[TC][RW] = reinterpret_cast<float (*)[TC][RW]>(s_buf);
  float2* s_off = reinterpret_cast<float2*>(s_buf);
  float4* s_acc = s_buf + threadIdx.x;   // NSL = 1: this lane's sums, s_acc[q * NTH]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sl = lane & 15, slot = lane >> 4;
  const int hs = sl >> 3, g = sl & 7;
  // NSL = 2: lanes g and 7 - g of a token's group hold the same two steps
  // 2hs, 2hs + 1; the lane keeps the softmax of step 2hs + par
  const int par = g >> 2;
  // this lane's token offset o within an iteration
  const int my = NSL == 2 ? wave * SPW + slot : (wave * SPW + slot) * 2 + hs;
  const int split = blockIdx.x;
  const int hq = blockIdx.y;
  const int h = hq / a.gqa;
  const int b = blockIdx.z / a.n_blk_serv;
  const int beta = a.blk0 + (blockIdx.z - b * a.n_blk_serv);
  const int t_lo = max(a.step0, beta * TC), t_hi = min(a.step0 + a.n_steps, (beta + 1) * TC);
  const int m0 = a.step0 - beta * TC;   // NSL = 1: the served step (n_steps = 1)
  // step of the lane's slot ml
  auto lane_step = [&](int ml) { return NSL == 2 ? 2 * hs + ml : m0; };

  // ---- codebooks -> LDS (fp16, step-major), power-of-two range scaling; the
  // bf16 sink and recent keys enter the transformed space times w, so their
  // range counts with that factor.  The effective-query coefficients satisfy
  // |A_o|, |B_o| <= |a| + |b| <= 2 max_d |q_d| / min(w_d, w_(d^D/2)), the
  // bound that sets their power-of-two scale (the coefficients carry the
  // softmax scale log2(e) / sqrt(D) as well).
  const int64_t cbo = ((int64_t)h * a.n_blk + beta) * a.K * G;
  const int r = tid;
  float kx[G], vx[G];
  float mq, mk, mv;
  decode_input_absmax(a, b, hq, 1, h, t_lo, t_hi, split == 0, a.w + h * D, mq, mk, mv);
  mq *= 2.f * a.qscale;
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
  if (tid == 0) s_prog = 0;   // read only after the next barrier
  // offset angles o * w_f, w_f = theta^(-2f/D), in fp32
  {
    const float l2t = log2f(a.theta);
    for (int x = tid; x < TPI * HD; x += NTH) {
      const int o = x / HD, f = x - o * HD;
      const float ang = (float)o * exp2f(-(float)(2 * f) / (float)D * l2t);
      float sn, cs;
      sincosf(ang, &sn, &cs);
      s_off[x] = make_float2(cs, sn);
    }
  }
  __syncthreads();
  mk = s_amax[0][0];
  mv = s_amax[1][0];
  mq = s_amax[2][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    mk = fmaxf(mk, s_amax[0][w]);
    mv = fmaxf(mv, s_amax[1][w]);
    mq = fmaxf(mq, s_amax[2][w]);
  }
  const int shk = pow2_range_shift(mk, 14), shv = pow2_range_shift(mv, kTVLim(NSL)), shq = pow2_range_shift(mq, 14);
  {
    const float sk = ldexpf(1.f, -shk), sv = ldexpf(1.f, -shv);
    uint32_t kw[2 * C], vw[2 * C];   // [m][pair]
#pragma unroll
    for (int m = 0; m < TC; ++m)
#pragma unroll
      for (int ip = 0; ip < DW; ++ip) {
        kw[m * DW + ip] = pack_h2t(kx[(2 * ip) * TC + m] * sk, kx[(2 * ip + 1) * TC + m] * sk);
        vw[m * DW + ip] = pack_h2t(vx[(2 * ip) * TC + m] * sv, vx[(2 * ip + 1) * TC + m] * sv);
      }
    if constexpr (kRep) {
      if (r < 256) {
        // the eight copies, stored in a lane-rotated order to spread the
        // stores over the banks
#pragma unroll
        for (int j0 = 0; j0 < 8; ++j0) {
          const int j = (j0 + r) & 7;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            cbk[r * kRowQ + 2 * j + u] = make_uint4(kw[4 * u], kw[4 * u + 1], kw[4 * u + 2], kw[4 * u + 3]);
            cbv[r * kRowQ + 2 * j + u] = make_uint4(vw[4 * u], vw[4 * u + 1], vw[4 * u + 2], vw[4 * u + 3]);
          }
        }
      }
    } else if constexpr (kSlice) {
      if (r < 256) {
        // step m0's slice of codeword r (DW = 2 dwords), sixteen copies
        auto pick = [&](const uint32_t (&x)[2 * C], int ip) {
          return m0 == 0 ? x[ip] : m0 == 1 ? x[DW + ip] : m0 == 2 ? x[2 * DW + ip] : x[3 * DW + ip];
        };
        const uint2 ks = make_uint2(pick(kw, 0), pick(kw, 1)), vs = make_uint2(pick(vw, 0), pick(vw, 1));
        uint2* row = reinterpret_cast<uint2*>(s_k + r * kRowQ);
#pragma unroll
        for (int j0 = 0; j0 < 16; ++j0) {
          const int j = (j0 + r) & 15;
          row[j] = ks;
          row[16 + j] = vs;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 2 * QW; ++u) {
        cbk[r * kRowQ + u] = make_uint4(kw[4 * u], kw[4 * u + 1], kw[4 * u + 2], kw[4 * u + 3]);
        cbv[r * kRowQ + u] = make_uint4(vw[4 * u], vw[4 * u + 1], vw[4 * u + 2], vw[4 * u + 3]);
      }
    }
  }

  // ---- effective-query coefficients A_o, B_o of this lane's channels
  // d' = 16g + j for its steps.  They enter fp16 times 2^-shq.
  uint32_t A2[NSL][NPR], B2[NSL][NPR];
  const float qsc = a.qscale * ldexpf(1.f, -shq);
  {
    int och[NCH];
    float rw[NCH];
    float2 oc[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int o = a.perm[h * D + NCH * g + j] & (D - 1);   // stays in bounds for any input
      och[j] = o;
      rw[j] = 1.f / a.w[h * D + o];
      oc[j] = s_off[my * HD + (o & (HD - 1))];
    }
#pragma unroll
    for (int ml = 0; ml < NSL; ++ml) {
      const int t = beta * TC + lane_step(ml);
      const bool act = t >= t_lo && t < t_hi;
      const uint16_t* qr = a.q + (((int64_t)b * a.Hq + hq) * a.n_steps + (act ? t - a.step0 : 0)) * D;
#pragma unroll
      for (int p = 0; p < NPR; ++p) {
        float av[2], bv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int j = 2 * p + u, o = och[j];
          const float qo = bf16_to_f32(qr[o]) * qsc;
          const float qp = bf16_to_f32(qr[o ^ HD]) * qsc;
          const float aa = qo * rw[j];
          const float bb = (o < HD ? qp : -qp) * rw[j];
          av[u] = act ? aa * oc[j].x + bb * oc[j].y : 0.f;
          bv[u] = act ? bb * oc[j].x - aa * oc[j].y : 0.f;
        }
        A2[ml][p] = pack_h2t(av[0], av[1]);
        B2[ml][p] = pack_h2t(bv[0], bv[1]);
      }
    }
  }
  // Scores are kept in units of 2^-E (E = shk + shq, the codebook and
  // coefficient scales): r = (dot product of the fp16 operands) * sigma, and
  // the true base-2 score is r * 2^E.  The running maximum mr is in the same
  // units, so score minus maximum is one mixed-precision fma (sigma in fp16)
  // and 2^E enters only the exponent.
  const int E = shk + shq;
  const float lagr = ldexpf((float)kTLag, -E);

  // running maximum and sum of weights of the lane's one softmax step (the
  // kept step with NSL = 2, the served step with NSL = 1)
  float mr[1] = {-INFINITY}, lrow[1] = {0.f};
  uint32_t acc16[NSL][NPR];
#pragma unroll
  for (int ml = 0; ml < NSL; ++ml)
#pragma unroll
    for (int p = 0; p < NPR; ++p) acc16[ml][p] = 0u;
  __syncthreads();   // codebooks staged; the offset table is no longer read
  // NSL = 2: the two float4 of the wave's sums that this lane adds into at a
  // flush: row slot of the wave takes step 2hs + (slot >> 1), channels
  // 16g + 8(slot & 1) .. +7 (the partials the cross-row reduction leaves
  // in this lane)
  float* const s_mine = &s_red[wave][2 * hs + (slot >> 1)][NCH * g + 8 * (slot & 1)];
  if constexpr (kShared) {
    reinterpret_cast<float4*>(s_mine)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    reinterpret_cast<float4*>(s_mine)[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  } else {
#pragma unroll
    for (int q = 0; q < kAccQ; ++q) s_acc[q * NTH] = make_float4(0.f, 0.f, 0.f, 0.f);
  }

  int nb = a.N;
  if (a.seq_len) nb = max(0, min(a.seq_len[b], a.N));
  const int tok_lo = split * a.tok_per_split;
  const int tok_hi = min(nb, tok_lo + a.tok_per_split);
  const int n_sink = split == 0 ? a.n_s : 0;
  const int n_rec = split == 0 ? a.n_r : 0;
  const int64_t irow0 = (((int64_t)b * a.H + h) * a.n_blk + beta) * (int64_t)a.N_cap;
  const int64_t sink0 = (((int64_t)b * a.H + h) * a.T + beta * TC) * (int64_t)a.n_s;
  const int64_t rec0 = (((int64_t)b * a.H + h) * a.T + beta * TC) * (int64_t)a.r_cap;
  const uint16_t* rope16 = reinterpret_cast<const uint16_t*>(a.rope);
  const float ksc = ldexpf(1.f, -shk), vsc = ldexpf(1.f, -shv);

  // Per-token loads go through buffer descriptors: the per-lane byte offset
  // is fixed, the iteration's offset is uniform (a scalar register), and an
  // offset past the described range reads 0 instead of faulting.
  const __amdgpu_buffer_rsrc_t rope_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)a.rope, 0, a.n_pos * D * 2, kBufWord3);
  // byte offsets in a table row of the aligned 4-byte words holding the
  // cosines of the two frequencies of the channel pair this lane loads (pair
  // lane / 8 of group lane % 8), each sine sitting 8 bytes after its cosine,
  // and the byte selector that packs the two fp16 values (a low, b high) out
  // of the two words
  int rope_a, rope_b;
  uint32_t rope_sel;
  {
    const int pg = lane & 7, pp = lane >> 3;
    const int fa = a.perm[h * D + NCH * pg + 2 * pp] & (HD - 1);
    const int fb = a.perm[h * D + NCH * pg + 2 * pp + 1] & (HD - 1);
    rope_a = (fa >> 1) * 4 + (fa >> 2) * 8;   // = ((fa >> 2) * 8 + (fa & 3)) * 2, rounded down to 4
    rope_b = (fb >> 1) * 4 + (fb >> 2) * 8;
    const uint32_t ba = 2 * (fa & 1), bb = 4 + 2 * (fb & 1);
    rope_sel = ba | (ba + 1) << 8 | bb << 16 | (bb + 1) << 24;
  }
  // (cos pair, sin pair) of this lane's channel pair at position P
  auto load_row = [&](int P) {
    const uint32_t ca = __builtin_amdgcn_raw_buffer_load_b32(rope_rs, rope_a, P * (D * 2), 0);
    const uint32_t cb = __builtin_amdgcn_raw_buffer_load_b32(rope_rs, rope_b, P * (D * 2), 0);
    const uint32_t sa = __builtin_amdgcn_raw_buffer_load_b32(rope_rs, rope_a, P * (D * 2) + 8, 0);
    const uint32_t sb = __builtin_amdgcn_raw_buffer_load_b32(rope_rs, rope_b, P * (D * 2) + 8, 0);
    return make_uint2(__builtin_amdgcn_perm(cb, ca, rope_sel), __builtin_amdgcn_perm(sb, sa, rope_sel));
  };
  // The wave's pair table for one position: written and read by this wave
  // only; LDS instructions of one wave execute in order, so the entries read
  // are this iteration's and the next write follows these reads.
  auto pair_table = [&](uint2 row, uint32_t (&cs2)[NPR], uint32_t (&sn2)[NPR]) {
    s_pair[wave][lane] = row;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int p = 0; p < NPR; ++p) {
      const uint2 e = s_pair[wave][8 * p + g];
      cs2[p] = e.x;
      sn2[p] = e.y;
    }
  };
  // Dot products of the lane's steps (summed over the 8 lanes of the
  // token's group, before sigma); Kw[k][ml*DW + ip] = pair slot k*DW + ip
  // (a channel pair of chunk slot k) at the lane's step ml.
  auto scores = [&](const uint32_t (&cs2)[NPR], const uint32_t (&sn2)[NPR], const uint32_t (&Kw)[NCK][KWD],
                    float (&sc)[NSL]) {
    // the two steps' chains interleave, so the dependent pk_mul -> pk_fma
    // -> dot2 sequences overlap
    float part[NSL];
#pragma unroll
    for (int p = 0; p < NPR; ++p) {
      h2t_t e2[NSL];
#pragma unroll
      for (int ml = 0; ml < NSL; ++ml) e2[ml] = as_h2t(A2[ml][p]) * as_h2t(cs2[p]);
#pragma unroll
      for (int ml = 0; ml < NSL; ++ml) e2[ml] = as_h2t(B2[ml][p]) * as_h2t(sn2[p]) + e2[ml];
#pragma unroll
      for (int ml = 0; ml < NSL; ++ml) {
        const h2t_t k2 = as_h2t(Kw[p / DW][ml * DW + p % DW]);
        part[ml] = p == 0 ? dot2_first(e2[ml], k2) : __builtin_amdgcn_fdot2(e2[ml], k2, part[ml], false);
      }
    }
    if constexpr (kShared) {
      // lanes g and 7 - g trade the step the other keeps, then the four
      // lanes of each half of the group add up (sc[0]: the kept step)
      const float keep = par ? part[1] : part[0], give = par ? part[0] : part[1];
      float x = keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(give), 0x141, 0xF, 0xF, true));
      x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
      x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
      sc[0] = x;
    } else {
#pragma unroll
      for (int ml = 0; ml < NSL; ++ml) sc[ml] = group_sum<8>(part[ml]);
    }
  };
  // fp16 partial sums into the fp32 sums in LDS.  NSL = 2: the four rows'
  // partials are first summed and scattered by two permlane swaps, after
  // which row r holds the words of step r >> 1, pairs 4(r & 1) .. +3, and
  // adds them into its two float4 of the wave's sums.  NSL = 1: channel
  // pairs 2p, 2p+1 are float4 (2p) / 4 of the lane's own sums, components
  // 2p % 4, +1.
  auto flush = [&]() {
    if constexpr (kShared) {
      uint32_t r1[NPR], f[NPR / 2];
#pragma unroll
      for (int j = 0; j < NPR; ++j) {
        const auto x = __builtin_amdgcn_permlane32_swap(acc16[0][j], acc16[1][j], false, false);
        r1[j] = __builtin_bit_cast(uint32_t, as_h2t(x[0]) + as_h2t(x[1]));
      }
#pragma unroll
      for (int j = 0; j < NPR / 2; ++j) {
        const auto x = __builtin_amdgcn_permlane16_swap(r1[j], r1[j + NPR / 2], false, false);
        f[j] = __builtin_bit_cast(uint32_t, as_h2t(x[0]) + as_h2t(x[1]));
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float4 v = reinterpret_cast<float4*>(s_mine)[u];
        add_f16x2(f[2 * u], v.x, v.y);
        add_f16x2(f[2 * u + 1], v.z, v.w);
        reinterpret_cast<float4*>(s_mine)[u] = v;
      }
    } else {
#pragma unroll
      for (int q = 0; q < kAccQ; ++q) {
        const int ml = q / (NCH / 4), p0 = 2 * (q % (NCH / 4));
        float4 v = s_acc[q * NTH];
        add_f16x2(acc16[ml][p0], v.x, v.y);
        add_f16x2(acc16[ml][p0 + 1], v.z, v.w);
        s_acc[q * NTH] = v;
      }
    }
#pragma unroll
    for (int ml = 0; ml < NSL; ++ml)
#pragma unroll
      for (int p = 0; p < NPR; ++p) acc16[ml][p] = 0u;
  };
  auto rescale = [&](float4* v, float alpha) {
    float4 x = *v;
    x.x *= alpha;
    x.y *= alpha;
    x.z *= alpha;
    x.w *= alpha;
    *v = x;
  };
  // A token whose score exceeds the running maximum by more than kTLag
  // raises the maximum and rescales every sum kept relative to it.
  // NSL = 2: sg.x is the sigma of the lane's kept step, sc[0] its score; the
  // maximum is raised for the four rows together, in a branch the whole wave
  // takes, and the weights of both steps reach the P*V update through the
  // partner lane 7 - g.  NSL = 1: sg.x is the served step's sigma.
  auto accumulate = [&](const float (&sc)[NSL], h2t_t sg, const uint32_t (&Vw)[NCK][KWD], bool valid) {
    const float sgm = (float)sg.x;
    float t = fmaf(sc[0], sgm, -mr[0]);   // (score - running maximum) * 2^-E
    if constexpr (kShared) {
      if (__builtin_amdgcn_ballot_w64(valid && t > lagr) != 0) {
        const float nm = fmaxf(mr[0], group4_max(valid ? sc[0] * sgm : -INFINITY));
        // some row holds a valid token here (the rows of a lane set are the
        // wave's four tokens, valid alike for every lane set), so nm is finite
        const float al = __builtin_amdgcn_exp2f(__builtin_amdgcn_ldexpf(mr[0] - nm, E));
        const float ao = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(al), 0x141, 0xF, 0xF, true));
        const float a0 = par ? ao : al, a1 = par ? al : ao;
        const h2t_t a20 = {(_Float16)a0, (_Float16)a0}, a21 = {(_Float16)a1, (_Float16)a1};
        lrow[0] *= al;
#pragma unroll
        for (int p = 0; p < NPR; ++p) {
          acc16[0][p] = __builtin_bit_cast(uint32_t, as_h2t(acc16[0][p]) * a20);
          acc16[NSL - 1][p] = __builtin_bit_cast(uint32_t, as_h2t(acc16[NSL - 1][p]) * a21);
        }
        const float ar = (slot >> 1) ? a1 : a0;
        rescale(reinterpret_cast<float4*>(s_mine), ar);
        rescale(reinterpret_cast<float4*>(s_mine) + 1, ar);
        mr[0] = nm;
        t = fmaf(sc[0], sgm, -nm);
      }
      if (!valid) return;
      const float pr = __builtin_amdgcn_exp2f(__builtin_amdgcn_ldexpf(t, E));
      lrow[0] += pr;
      const uint32_t p16 = __builtin_bit_cast(uint16_t, (_Float16)pr);
      const uint32_t o16 = __builtin_amdgcn_mov_dpp(p16, 0x141, 0xF, 0xF, true);
      // (own, partner's) is the order (step 2hs, step 2hs + 1) for lanes
      // g < 4; lanes g >= 4 (banks 1 and 3 of each row of 16) take their
      // partner's word instead
      const uint32_t x = __builtin_amdgcn_perm(o16, p16, 0x05040100u);
      const h2t_t pp = as_h2t(__builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xA, false));
      const h2t_t p0 = {pp.x, pp.x}, p1 = {pp.y, pp.y};
#pragma unroll
      for (int p = 0; p < NPR; ++p) {
        acc16[0][p] = __builtin_bit_cast(uint32_t, as_h2t(Vw[p / DW][p % DW]) * p0 + as_h2t(acc16[0][p]));
        acc16[NSL - 1][p] = __builtin_bit_cast(
            uint32_t, as_h2t(Vw[p / DW][(NSL - 1) * DW + p % DW]) * p1 + as_h2t(acc16[NSL - 1][p]));
      }
    } else {
      if (!valid) return;
      if (t > lagr) {
        const float alpha = __builtin_amdgcn_exp2f(__builtin_amdgcn_ldexpf(-t, E));
        const h2t_t a2 = {(_Float16)alpha, (_Float16)alpha};
        lrow[0] *= alpha;
#pragma unroll
        for (int q = 0; q < NCH / 4; ++q) rescale(&s_acc[q * NTH], alpha);
#pragma unroll
        for (int p = 0; p < NPR; ++p) acc16[0][p] = __builtin_bit_cast(uint32_t, as_h2t(acc16[0][p]) * a2);
        mr[0] = sc[0] * sgm;
        t = 0.f;
      }
      const float pr = __builtin_amdgcn_exp2f(__builtin_amdgcn_ldexpf(t, E));
      lrow[0] += pr;
      const h2t_t p2 = {(_Float16)pr, (_Float16)pr};
#pragma unroll
      for (int p = 0; p < NPR; ++p)
        acc16[0][p] = __builtin_bit_cast(uint32_t, as_h2t(Vw[p / DW][p % DW]) * p2 + as_h2t(acc16[0][p]));
    }
  };

  // ---- bf16 items (split 0): sinks at positions 0..n_s-1, then the recent
  // window at n_s + N_b + r.  Their keys are raw, so they enter the
  // transformed space as w[p(d')] * k[p(d')] with sigma = 1.  Item base + o
  // of a run sits at position P0 + base + o.
  auto bf16_items = [&](int count, int P0, bool is_rec) {
    for (int base = 0; base < count; base += TPI) {
      const int it = base + my;
      const bool valid = it < count;
      const int itc = valid ? it : 0;
      uint32_t cs2[NPR], sn2[NPR];
      pair_table(load_row(P0 + base), cs2, sn2);
      uint32_t Kw[NCK][KWD], Vw[NCK][KWD];
#pragma unroll
      for (int ml = 0; ml < NSL; ++ml) {
        const int m = lane_step(ml);
        const uint16_t* kr = is_rec ? a.rk + (rec0 + (int64_t)m * a.r_cap + itc) * D
                                    : a.sk + (sink0 + (int64_t)m * a.n_s + itc) * D;
        const uint16_t* vr = is_rec ? a.rv + (rec0 + (int64_t)m * a.r_cap + itc) * D
                                    : a.sv + (sink0 + (int64_t)m * a.n_s + itc) * D;
#pragma unroll
        for (int p = 0; p < NPR; ++p) {
          float z[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int o = a.perm[h * D + NCH * g + 2 * p + u] & (D - 1);
            z[u] = bf16_to_f32(kr[o]) * a.w[h * D + o] * ksc;
          }
          const uint32_t vv = *reinterpret_cast<const uint32_t*>(vr + NCH * g + 2 * p);
          Kw[p / DW][ml * DW + p % DW] = pack_h2t(z[0], z[1]);
          Vw[p / DW][ml * DW + p % DW] = pack_h2t(bf16lo(vv) * vsc, bf16hi(vv) * vsc);
        }
      }
      const h2t_t one2 = {(_Float16)1.f, (_Float16)1.f};
      float sc[NSL];
      scores(cs2, sn2, Kw, sc);
      accumulate(sc, one2, Vw, valid);
      flush();
    }
  };
  if (n_sink > 0) bf16_items(n_sink, 0, false);
  if (n_rec > 0) bf16_items(n_rec, a.n_s + nb, true);

  // ---- quantized tokens, one per lane slot per iteration; index words,
  // sigma and the table row of the next iteration are loaded one iteration
  // ahead.
  const int n_tok = max(0, tok_hi - tok_lo);
  const int P0 = a.n_s + tok_lo;
  // word of the index row holding this lane's index bytes, and their bit offset
  const int kwo = C == 4 ? g : (g >> 1);
  const int kbit = C == 4 ? 0 : 16 * (g & 1);
  // c = 8: byte selector spreading the lane's two index bytes into 16-bit halves
  const uint32_t isel = (uint32_t)(kbit / 8) | 0x0C00u | (uint32_t)(kbit / 8 + 1) << 16 | 0x0C000000u;
  // byte offset of the lane's half inside a codeword row: half hs of its
  // group's copy (kRep) or of the one copy
  const uint32_t hsb = kRep ? g * 32 + hs * 16 : hs * QW * 16;
  constexpr int kRow = kRowQ * 16;   // bytes per codeword row in LDS
  const uint32_t hsbv = hsb + 65536u;   // kRep: the V rows follow 64 KB on
  const uint32_t slb = 8u * sl;          // kSlice: the lane's copy of a K slice
  // index rows of this (batch, kv-head, block) and sigma of this batch entry;
  // a lane past the split's last token reads a later row or 0 (unused)
  const __amdgpu_buffer_rsrc_t kid_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.kidx + irow0 * CPT), 0, a.N_cap * CPT, kBufWord3);
  const __amdgpu_buffer_rsrc_t vid_rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.vidx + irow0 * CPT), 0, a.N_cap * CPT, kBufWord3);
  const __amdgpu_buffer_rsrc_t sig_rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.sigma + (int64_t)b * a.sig_cap * a.T), 0, a.sig_cap * a.T * 2, kBufWord3);
  const int idx_lane = (tok_lo + my) * CPT + 4 * kwo;
  // sigma of the lane's steps: one 4-byte word holds an even step and the next
  // sigma: NSL = 2, the lane's kept step (2 bytes); NSL = 1, the 4-byte word
  // holding the served step and its even/odd neighbour
  const int sig_lane = ((tok_lo + my) * a.T + beta * TC + (NSL == 2 ? 2 * hs + par : (m0 & ~1))) * 2;
  // what one iteration loads ahead: index words, sigma and the table row
  struct Ahead {
    uint32_t kw, vw, sg;
    uint2 row;
  };
  auto load_ahead = [&](int base) {
    Ahead x;
    x.kw = __builtin_amdgcn_raw_buffer_load_b32(kid_rs, idx_lane, base * CPT, 0);
    x.vw = __builtin_amdgcn_raw_buffer_load_b32(vid_rs, idx_lane, base * CPT, 0);
    if constexpr (NSL == 2)
      x.sg = __builtin_amdgcn_raw_buffer_load_b16(sig_rs, sig_lane, base * a.T * 2, 0);
    else
      x.sg = __builtin_amdgcn_raw_buffer_load_b32(sig_rs, sig_lane, base * a.T * 2, 0);
    x.row = load_row(P0 + (base < n_tok ? base : 0));         // a row of this split's tokens
    return x;
  };
  auto iteration = [&](int base, int it, const Ahead& cur) {
    const bool valid = my < n_tok - base;   // one compare with a scalar bound
    // LDS order: the pair table, then the K gathers, then the V gathers, so
    // the scores can start while the V gathers are in flight
    uint32_t cs2[NPR], sn2[NPR];
    pair_table(cur.row, cs2, sn2);
    uint32_t Kw[NCK][KWD], Vw[NCK][KWD];
    // codeword dwords of the lane's steps: the half hs (both steps), or the
    // served step's dwords
    if constexpr (kRep) {
      // offset of the codeword half: bytes (hsb byte 0, index byte k, hsb
      // byte 2, 0), hsbv for V
      auto gather = [&](uint32_t w, uint32_t base, int k, uint32_t (&out)[KWD]) {
        const uint32_t o = __builtin_amdgcn_perm(w, base, 0x0C020000u | (uint32_t)(4 + k) << 8);
        const uint4 y = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(s_k) + o);
        out[0] = y.x; out[1] = y.y; out[2] = y.z; out[3] = y.w;
      };
#pragma unroll
      for (int k = 0; k < NCK; ++k) gather(cur.kw, hsb, k, Kw[k]);
#pragma unroll
      for (int k = 0; k < NCK; ++k) gather(cur.vw, hsbv, k, Vw[k]);
    } else if constexpr (kSlice) {
      // offset of the step slice: bytes (8 (lane mod 16) (+ 128 for V), index
      // byte k, 0, 0)
      auto gather = [&](uint32_t w, uint32_t base, int k, uint32_t (&out)[KWD]) {
        const uint32_t o = __builtin_amdgcn_perm(w, base, 0x0C0C0000u | (uint32_t)(4 + k) << 8);
        const uint2 y = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(s_k) + o);
        out[0] = y.x; out[1] = y.y;
      };
#pragma unroll
      for (int k = 0; k < NCK; ++k) gather(cur.kw, slb, k, Kw[k]);
#pragma unroll
      for (int k = 0; k < NCK; ++k) gather(cur.vw, slb + 128u, k, Vw[k]);
    } else if constexpr (NSL == 2) {
      // (c = 8) The lane's two index bytes are spread into the 16-bit halves
      // of one word, so each codeword's byte offset, idx * 32 QW + the half's
      // 16 QW hs, is one multiply-add on a half.
      const uint32_t kh[2] = {__builtin_amdgcn_perm(cur.kw, cur.kw, isel), 0u};
      const uint32_t vh[2] = {__builtin_amdgcn_perm(cur.vw, cur.vw, isel), 0u};
      auto gather = [&](const uint4* cb, uint32_t off, uint32_t (&out)[KWD]) {
        const uint4* x = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(cb) + off);
#pragma unroll
        for (int u = 0; u < QW; ++u) {
          const uint4 y = x[u];
          out[4 * u] = y.x; out[4 * u + 1] = y.y; out[4 * u + 2] = y.z; out[4 * u + 3] = y.w;
        }
      };
      static_assert(NCK == 2, "the spread form serves c = 8");
      gather(cbk, mad_half<0, kRow>(kh[0], hsb), Kw[0]);
      gather(cbk, mad_half<1, kRow>(kh[0], hsb), Kw[1]);
      gather(cbv, mad_half<0, kRow>(vh[0], hsb), Vw[0]);
      gather(cbv, mad_half<1, kRow>(vh[0], hsb), Vw[1]);
    } else {
      // the served step's DW dwords inside its half
      auto gather = [&](const uint4* cb, uint32_t idx, uint32_t (&out)[KWD]) {
        const uint32_t* w = reinterpret_cast<const uint32_t*>(cb + (2 * idx + (m0 >> 1)) * QW) + (m0 & 1) * DW;
        if constexpr (DW == 2) {
          const uint2 x = *reinterpret_cast<const uint2*>(w);
          out[0] = x.x; out[1] = x.y;
        } else {
          const uint4 x = *reinterpret_cast<const uint4*>(w);
          out[0] = x.x; out[1] = x.y; out[2] = x.z; out[3] = x.w;
        }
      };
#pragma unroll
      for (int k = 0; k < NCK; ++k) gather(cbk, __builtin_amdgcn_ubfe(cur.kw, kbit + 8 * k, 8), Kw[k]);
#pragma unroll
      for (int k = 0; k < NCK; ++k) gather(cbv, __builtin_amdgcn_ubfe(cur.vw, kbit + 8 * k, 8), Vw[k]);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep every gather issued ahead of the arithmetic
    h2t_t s16 = as_h2t(cur.sg);
    if constexpr (NSL == 1) s16.x = (m0 & 1) ? s16.y : s16.x;
    float sc[NSL];
    scores(cs2, sn2, Kw, sc);
    accumulate(sc, s16, Vw, valid);
    // every kFl iterations (it is the same in every lane): the flush, and
    // the wave's priority from its progress against the workgroup's
    if ((it & (kFl - 1)) == kFl - 1) {
      flush();
      int tot = 0;
      if (lane == 0) tot = atomicAdd(&s_prog, 1) + 1;
      tot = __builtin_amdgcn_readfirstlane(tot);
      if (((it + 1) / kFl) * NW < tot)
        __builtin_amdgcn_s_setprio(2);
      else
        __builtin_amdgcn_s_setprio(0);
    }
  };
  // two iterations per trip, loading into alternate register sets, so that
  // nothing loaded ahead is copied from one set to the other
  if (n_tok > 0) {
    Ahead x0 = load_ahead(0), x1;
    for (int base = 0, it = 0;; base += 2 * TPI, it += 2) {
      x1 = load_ahead(base + TPI);
      iteration(base, it, x0);
      if (base + TPI >= n_tok) break;
      x0 = load_ahead(base + 2 * TPI);
      iteration(base + TPI, it + 1, x1);
      if (base + 2 * TPI >= n_tok) break;
    }
  }
  __builtin_amdgcn_s_setprio(0);
  flush();
  if constexpr (kShared) {
    // the sums are already the wave's merge slot; its maximum is the rows'
    // common one, its sum of weights the rows' total (lanes g = 0 and 4 of
    // row 0 hold steps 2hs and 2hs + 1)
    const float l = group4_sum(lrow[0]);
    if (slot == 0 && (g & 3) == 0) {
      s_red[wave][2 * hs + par][D] = __builtin_amdgcn_ldexpf(mr[0], E);
      s_red[wave][2 * hs + par][D + 1] = l;
    }
  } else {
    float acc[NSL][NCH];
#pragma unroll
    for (int q = 0; q < kAccQ; ++q) {
      const float4 v = s_acc[q * NTH];
      const int ml = q / (NCH / 4), j0 = 4 * (q % (NCH / 4));
      acc[ml][j0] = v.x;
      acc[ml][j0 + 1] = v.y;
      acc[ml][j0 + 2] = v.z;
      acc[ml][j0 + 3] = v.w;
    }
    __syncthreads();   // every lane holds its sums: the region becomes the merge buffer
    // running maxima back to base-2 score units
    float mrow[NSL];
#pragma unroll
    for (int ml = 0; ml < NSL; ++ml) mrow[ml] = __builtin_amdgcn_ldexpf(mr[ml], E);

    // ---- merge the lanes of the wave that hold the same channel and step
    // (equal g)
#pragma unroll
    for (int off = LPT / 2; off < kWave; off <<= 1) {
#pragma unroll
      for (int ml = 0; ml < NSL; ++ml) {
        const float om = __shfl_xor(mrow[ml], off);
        const float ol = __shfl_xor(lrow[ml], off);
        const float mm = fmaxf(mrow[ml], om);
        const float a1 = mrow[ml] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrow[ml] - mm);
        const float a2 = om == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(om - mm);
        lrow[ml] = lrow[ml] * a1 + ol * a2;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
          const float oa = __shfl_xor(acc[ml][j], off);
          acc[ml][j] = acc[ml][j] * a1 + oa * a2;
        }
        mrow[ml] = mm;
      }
    }
    if ((lane >> 3) == 0) {
#pragma unroll
      for (int ml = 0; ml < NSL; ++ml) {
        const int m = lane_step(ml);
#pragma unroll
        for (int j = 0; j < NCH; ++j) s_red[wave][m][NCH * g + j] = acc[ml][j];
        if (g == 0) {
          s_red[wave][m][D] = mrow[ml];
          s_red[wave][m][D + 1] = lrow[ml];
        }
      }
    }
  }
  __syncthreads();
  const float osc = ldexpf(1.f, shv);
  // one split (out set): the rows go straight to out / lse, since the merge
  // of a single partial returns it unchanged
  const bool direct = a.out != nullptr;
  for (int x = tid; x < TC * D; x += NTH) {
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
    const int64_t row = ((int64_t)b * a.Hq + hq) * a.n_steps + (t - a.step0);
    const float o = den > 0.f ? num / den * osc : 0.f;
    const float l = den > 0.f ? (mm + __log2f(den)) * 0.69314718055994531f : -INFINITY;
    if (direct) {
      a.out[row * D + d] = o;
      if (d == 0 && a.lse) a.lse[row] = l;
    } else {
      float* dst = a.ws + (row * a.n_split + split) * (D + 1);
      dst[d] = o;
      if (d == 0) dst[D] = l;
    }
  }
}

hipError_t launch_decode_tasq(int G, bool one, const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.Hq, a.B * a.n_blk_serv);
  if (one && a.n_steps != 1) return hipErrorInvalidValue;
  if (G == 16 && one)
    hipLaunchKernelGGL((decode_tasq_kernel<4, 1>), grid, dim3(tasq_threads(4, 1)), 0, s, a);
  else if (G == 16)
    hipLaunchKernelGGL((decode_tasq_kernel<4, 2>), grid, dim3(tasq_threads(4, 2)), 0, s, a);
  else if (G == 32 && one)
    hipLaunchKernelGGL((decode_tasq_kernel<8, 1>), grid, dim3(tasq_threads(8, 1)), 0, s, a);
  else if (G == 32)
    hipLaunchKernelGGL((decode_tasq_kernel<8, 2>), grid, dim3(tasq_threads(8, 2)), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace loopvq
