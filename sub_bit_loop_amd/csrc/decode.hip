// LoopVQ fused decode attention over the compressed cache.
//
// LoopVQ review (arXiv 2611.05304), section 3.4 step 3: the kernel keeps the
// codebook in on-chip memory, looks each token's keys and values up by index,
// rotates the restored keys (RoPE after dequant, section 3.1) from a
// precomputed per-position sin/cos table, and combines context splits through
// their log-sum-exp (Flash-Decoding).  Section 3.1 eq. (5): step m of a block
// reads coordinate i*T_c + m of the shared codeword for channel q*c + i, so
// one index row serves every step of its block.
//
// Work decomposition (one workgroup = one batch entry, kv-head, block, q-head
// pass and context split; 4 waves):
//   * The block's K and V codebooks (bf16 [K][G]) sit in LDS.
//   * A token is served by LPT = (D/2)/c lanes.  Lane sl owns chunks sl and
//     sl + LPT, i.e. channels [c*sl, c*sl+c) and their RoPE partners
//     [D/2 + c*sl, ...); it gathers those codewords once and uses them for
//     all T_c steps of the block and every q-head of the pass.
//   * Partial dot products are summed over the LPT lanes with DPP; each lane
//     keeps an online softmax (running max / sum, base 2) and fp32 output
//     accumulators for its channels.
//   * Slots, then waves, are merged by log-sum-exp; each split writes a
//     normalised partial (out, lse) that the merge kernel combines.
// Sinks (bf16, pre-RoPE, positions 0..n_s-1) go through the same softmax in
// split 0.  With the channel pre-transform, keys are scored against an
// effective query (R_{-pos} q)[p(d')] / w[p(d')] and scaled by the token's
// sigma, which equals scoring the inverse-transformed, rotated key.
#include "common.h"
#include "kernels.h"

namespace loopvq {

template <int G, int TC, bool TASQ>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(DecodeArgs a) {
  constexpr int D = 128;
  constexpr int HD = D / 2;
  constexpr int C = G / TC;            // channels per step per code
  constexpr int CPT = D / C;           // index bytes per token row
  constexpr int LPT = HD / C;          // lanes per token
  constexpr int SPW = kWave / LPT;     // token slots per wave
  constexpr int NW = kDecodeThreads / kWave;
  constexpr int R = TC;                // rows per pass: steps of the block (one q-head)
  constexpr int NE = 2 * C;            // channels owned per lane
  __shared__ __attribute__((aligned(16))) uint16_t s_k[256 * G];
  __shared__ __attribute__((aligned(16))) uint16_t s_v[256 * G];
  __shared__ float s_red[NW][R][D + 2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sl = lane % LPT, slot = lane / LPT;
  const int split = blockIdx.x;
  const int h = blockIdx.y / a.gqa;
  const int hq = blockIdx.y;                 // one q-head per workgroup
  const int b = blockIdx.z / a.n_blk_serv;
  const int beta = a.blk0 + (blockIdx.z - b * a.n_blk_serv);

  {
    const int64_t cbo = ((int64_t)h * a.n_blk + beta) * a.K * G;
    const uint4* gk = reinterpret_cast<const uint4*>(a.kcb + cbo);
    const uint4* gv = reinterpret_cast<const uint4*>(a.vcb + cbo);
    uint4* lk = reinterpret_cast<uint4*>(s_k);
    uint4* lv = reinterpret_cast<uint4*>(s_v);
    const int n16 = a.K * G / 8;
    for (int e = tid; e < n16; e += kDecodeThreads) {
      lk[e] = gk[e];
      lv[e] = gv[e];
    }
  }

  // Rows of this pass: step t = beta*T_c + m for q-head hq.
  const int t_lo = max(a.step0, beta * TC), t_hi = min(a.step0 + a.n_steps, (beta + 1) * TC);
  float qa[R][NE], qb[R][NE];            // plain: qa = channel value, qb unused
  int freq[NE];
  float wch[NE];
  int och[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    const int p = e / C, i = e % C;
    const int dprime = p * HD + C * sl + i;   // transformed (or plain) channel
    int o = dprime;
    float wv = 1.f;
    if constexpr (TASQ) {
      o = a.perm[h * D + dprime] & (D - 1);   // stays in bounds for any input
      wv = a.w[h * D + o];
    }
    och[e] = o;
    wch[e] = wv;
    freq[e] = o & (HD - 1);
  }
#pragma unroll
  for (int m = 0; m < R; ++m) {
    const int t = beta * TC + m;
    const bool act = t >= t_lo && t < t_hi;
    const uint16_t* qr = a.q + (((int64_t)b * a.Hq + hq) * a.n_steps + (act ? t - a.step0 : 0)) * D;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int o = och[e];
      if constexpr (!TASQ) {
        qa[m][e] = act ? bf16_to_f32(qr[o]) * a.qscale : 0.f;
        qb[m][e] = 0.f;
      } else {
        const int partner = o ^ HD;
        const float sgn = o < HD ? 1.f : -1.f;
        qa[m][e] = act ? bf16_to_f32(qr[o]) * a.qscale / wch[e] : 0.f;
        qb[m][e] = act ? sgn * bf16_to_f32(qr[partner]) * a.qscale / wch[e] : 0.f;
      }
    }
  }

  float mrow[R], lrow[R], acc[R][NE];
#pragma unroll
  for (int m = 0; m < R; ++m) {
    mrow[m] = -INFINITY;
    lrow[m] = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[m][e] = 0.f;
  }
  __syncthreads();

  int nb = a.N;
  if (a.seq_len) nb = max(0, min(a.seq_len[b], a.N));
  const int tok_lo = split * a.tok_per_split;
  const int tok_hi = min(nb, tok_lo + a.tok_per_split);
  // bf16 items (sinks, then the recent window) are served by split 0.
  const int n_sink = split == 0 ? a.n_s : 0;
  const int n_bf = n_sink + (split == 0 ? a.n_r : 0);
  const int n_items = n_bf + max(0, tok_hi - tok_lo);
  const int64_t irow0 = (((int64_t)b * a.H + h) * a.n_blk + beta) * (int64_t)a.N_cap;
  const int64_t sink0 = (((int64_t)b * a.H + h) * a.T + beta * TC) * (int64_t)a.n_s;
  const int64_t rec0 = (((int64_t)b * a.H + h) * a.T + beta * TC) * (int64_t)a.r_cap;

  for (int base = 0; base < n_items; base += NW * SPW) {
    const int item = base + wave * SPW + slot;
    const bool valid = item < n_items;
    const int it = valid ? item : 0;
    const bool is_sink = it < n_bf;
    const bool is_rec = is_sink && it >= n_sink;
    const int j = is_sink ? 0 : tok_lo + it - n_bf;
    const int pos = !is_sink ? a.n_s + j : (is_rec ? a.n_s + nb + (it - n_sink) : it);

    float kv[NE][TC], vv[NE][TC], sg[TC];
    if (is_sink) {
#pragma unroll
      for (int m = 0; m < TC; ++m) {
        const uint16_t* kr = is_rec ? a.rk + (rec0 + (int64_t)m * a.r_cap + (it - n_sink)) * D
                                    : a.sk + (sink0 + (int64_t)m * a.n_s + it) * D;
        const uint16_t* vr = is_rec ? a.rv + (rec0 + (int64_t)m * a.r_cap + (it - n_sink)) * D
                                    : a.sv + (sink0 + (int64_t)m * a.n_s + it) * D;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const int p = e / C, i = e % C;
          kv[e][m] = bf16_to_f32(kr[och[e]]) * wch[e];
          vv[e][m] = bf16_to_f32(vr[p * HD + C * sl + i]);
        }
        sg[m] = 1.f;
      }
    } else {
      const uint8_t* kr = a.kidx + (irow0 + j) * CPT;
      const uint8_t* vr = a.vidx + (irow0 + j) * CPT;
      uint32_t ka[2] = {kr[sl], kr[sl + LPT]};
      uint32_t va[2] = {vr[sl], vr[sl + LPT]};
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        uint32_t kw[G / 2], vw[G / 2];
        const uint4* lk = reinterpret_cast<const uint4*>(s_k + ka[p] * G);
        const uint4* lv = reinterpret_cast<const uint4*>(s_v + va[p] * G);
#pragma unroll
        for (int c4 = 0; c4 < G / 8; ++c4) {
          uint4 x = lk[c4], y = lv[c4];
          kw[4 * c4 + 0] = x.x; kw[4 * c4 + 1] = x.y; kw[4 * c4 + 2] = x.z; kw[4 * c4 + 3] = x.w;
          vw[4 * c4 + 0] = y.x; vw[4 * c4 + 1] = y.y; vw[4 * c4 + 2] = y.z; vw[4 * c4 + 3] = y.w;
        }
#pragma unroll
        for (int i = 0; i < C; ++i) {
#pragma unroll
          for (int m = 0; m < TC; ++m) {
            const int u = i * TC + m;
            const uint32_t wk = kw[u >> 1], wvv = vw[u >> 1];
            kv[p * C + i][m] = (u & 1) ? bf16hi(wk) : bf16lo(wk);
            vv[p * C + i][m] = (u & 1) ? bf16hi(wvv) : bf16lo(wvv);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < TC; ++m) {
        if constexpr (TASQ) {
          const uint16_t sb = a.sigma[((int64_t)b * a.sig_cap + j) * a.T + beta * TC + m];
          sg[m] = (float)f16_bits_to_f64(sb);
        } else {
          sg[m] = 1.f;
        }
      }
    }

    // cos/sin of the token position for this lane's frequencies (fp16 table:
    // per position 16 quads of [cos f..f+3, sin f..f+3]).
    float cs[NE], sn[NE];
    const _Float16* rp = reinterpret_cast<const _Float16*>(a.rope) + (int64_t)pos * D;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int f = freq[e];
      cs[e] = (float)rp[(f >> 2) * 8 + (f & 3)];
      sn[e] = (float)rp[(f >> 2) * 8 + 4 + (f & 3)];
    }

    float sc[R];
#pragma unroll
    for (int m = 0; m < R; ++m) {
      float part = 0.f;
      if constexpr (!TASQ) {
#pragma unroll
        for (int i = 0; i < C; ++i) {
          const float k1 = kv[i][m], k2 = kv[C + i][m];
          const float k1r = k1 * cs[i] - k2 * sn[i];
          const float k2r = k2 * cs[i] + k1 * sn[i];
          part = fmaf(qa[m][i], k1r, part);
          part = fmaf(qa[m][C + i], k2r, part);
        }
      } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          const float u = qa[m][e] * cs[e] + qb[m][e] * sn[e];
          part = fmaf(kv[e][m], u, part);
        }
      }
      sc[m] = group_sum<LPT>(part) * sg[m];
    }

    if (valid) {
#pragma unroll
      for (int m = 0; m < R; ++m) {
        const float s = sc[m];
        if (s > mrow[m]) {
          const float alpha = __builtin_amdgcn_exp2f(mrow[m] - s);
          lrow[m] *= alpha;
#pragma unroll
          for (int e = 0; e < NE; ++e) acc[m][e] *= alpha;
          mrow[m] = s;
        }
        const float p = __builtin_amdgcn_exp2f(s - mrow[m]);
        lrow[m] += p;
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[m][e] = fmaf(p, vv[e][m], acc[m][e]);
      }
    }
  }

  // Merge the SPW slots of the wave (lanes with equal sl).
#pragma unroll
  for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
    for (int m = 0; m < R; ++m) {
      const float om = __shfl_xor(mrow[m], off);
      const float ol = __shfl_xor(lrow[m], off);
      const float mm = fmaxf(mrow[m], om);
      const float a1 = mrow[m] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrow[m] - mm);
      const float a2 = om == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(om - mm);
      lrow[m] = lrow[m] * a1 + ol * a2;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const float oa = __shfl_xor(acc[m][e], off);
        acc[m][e] = acc[m][e] * a1 + oa * a2;
      }
      mrow[m] = mm;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int m = 0; m < R; ++m) {
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int p = e / C, i = e % C;
        s_red[wave][m][p * HD + C * sl + i] = acc[m][e];
      }
      if (sl == 0) {
        s_red[wave][m][D] = mrow[m];
        s_red[wave][m][D + 1] = lrow[m];
      }
    }
  }
  __syncthreads();
  for (int x = tid; x < R * D; x += kDecodeThreads) {
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
    dst[d] = den > 0.f ? num / den : 0.f;
    if (d == 0) dst[D] = den > 0.f ? (mm + __log2f(den)) * 0.69314718055994531f : -INFINITY;
  }
}

__global__ __launch_bounds__(128) void merge_kernel(MergeArgs a) {
  constexpr int D = 128;
  const int row = blockIdx.x, d = threadIdx.x;
  const float* base = a.ws + (int64_t)row * a.n_split * (D + 1);
  float mx = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) mx = fmaxf(mx, base[s * (D + 1) + D]);
  float num = 0.f, den = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < a.n_split; ++s) {
      const float l = base[s * (D + 1) + D];
      const float wgt = l == -INFINITY ? 0.f : expf(l - mx);
      num += wgt * base[s * (D + 1) + d];
      den += wgt;
    }
  }
  a.out[(int64_t)row * D + d] = den > 0.f ? num / den : 0.f;
  if (d == 0 && a.lse) a.lse[row] = den > 0.f ? mx + logf(den) : -INFINITY;
}

template <int G, int TC>
static hipError_t dec_launch_s(bool tasq, const DecodeArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.Hq, a.B * a.n_blk_serv);
  if (tasq)
    hipLaunchKernelGGL((decode_kernel<G, TC, true>), grid, dim3(kDecodeThreads), 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<G, TC, false>), grid, dim3(kDecodeThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(int G, int TC, bool tasq, const DecodeArgs& a, hipStream_t s) {
  if (G == 16) {
    switch (TC) {
      case 1: return dec_launch_s<16, 1>(tasq, a, s);
      case 2: return dec_launch_s<16, 2>(tasq, a, s);
      case 4: return dec_launch_s<16, 4>(tasq, a, s);
      case 8: return dec_launch_s<16, 8>(tasq, a, s);
    }
  } else if (G == 32) {
    switch (TC) {
      case 1: return dec_launch_s<32, 1>(tasq, a, s);
      case 2: return dec_launch_s<32, 2>(tasq, a, s);
      case 4: return dec_launch_s<32, 4>(tasq, a, s);
      case 8: return dec_launch_s<32, 8>(tasq, a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(a.rows), dim3(128), 0, s, a);
  return hipGetLastError();
}

// fp64 angles rounded once to fp16 (review section 3.4: a precomputed
// per-position sin/cos table).  Layout per position: D/8 quads, each
// [cos f, cos f+1, cos f+2, cos f+3, sin f, ..., sin f+3] with f = 4 * quad.
__global__ void rope_table_kernel(double theta, int D, int n_pos, uint16_t* table) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int half = D / 2;
  if (x >= (int64_t)n_pos * half) return;
  const int p = (int)(x / half), f = (int)(x - (int64_t)p * half);
  const double omega = pow(theta, -2.0 * (double)f / (double)D);
  const double phi = (double)p * omega;
  uint16_t* row = table + (int64_t)p * D + (f >> 2) * 8;
  row[f & 3] = f64_to_f16_rne(cos(phi));
  row[4 + (f & 3)] = f64_to_f16_rne(sin(phi));
}

hipError_t launch_rope_table(double theta, int D, int n_pos, void* table, hipStream_t s) {
  const int64_t n = (int64_t)n_pos * (D / 2);
  const int threads = 256;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + threads - 1) / threads)), dim3(threads), 0, s,
                     theta, D, n_pos, static_cast<uint16_t*>(table));
  return hipGetLastError();
}

}  // namespace loopvq
