// Causal attention of every position after the sinks over the compressed
// cache, and its backward pass into the queries and the codebook entries:
// the hot part of loop-aware codebook fine-tuning.
//
// LoopVQ review (arXiv 2611.05304), section 3.2 eq. (6): the objective is the
// KL between the model's outputs with the precise cache and with the cache
// rebuilt from the codebooks, over the N positions after the bf16 sinks, with
// all T_c steps reading the rebuilt cache; the codebook entries get exact
// gradients by backpropagation (the argmin itself is not differentiated).
// Section 3.1 eq. (5): step m of a block reads coordinate i*T_c + m of the
// shared codeword; RoPE is applied after the dequant (section "terms").
//
// Query i of step t sits at position n_s + i and attends to the n_s sinks
// (positions 0..n_s-1, bf16, pre-RoPE) and to the tokens j <= i (position
// n_s + j).  Everything is fp32; the RoPE table is fp32 (cos, sin) per
// (position, frequency), computed in fp64.
//
// The same kernels, instantiated with C = 0, read a precise bf16 cache
// (every step's keys and values as stored) instead of codebook entries, and
// their key-side backward writes the gradient of every cached key (before
// RoPE) and value: the gradients the importance weights of the codebook
// k-means (eq. 3) are made of.
//
// All three products run on fp32 matrix cores (v_mfma_f32_32x32x2f32), so the
// arithmetic is fp32 as in a vector implementation.  Each wave owns 32 rows
// (queries, or tokens in the key-side passes) and works on LDS tiles of 32
// keys or queries; the operand layouts are described with each kernel.
#include "common.h"
#include "kernels.h"

namespace loopvq {

namespace {

constexpr int kPD = 128;              // head dimension
constexpr int kPH = 64;               // RoPE pairs
constexpr int kTile = 32;             // keys (or queries) staged per LDS tile
constexpr int kLds = kPD + 4;         // padded LDS row

// Stage step m's slice of the K and V codebooks of (kv-head h, block beta)
// as fp32 [K][C].
template <int C>
__device__ void stage_codebooks(const PrefillArgs& a, int h, int beta, int m, float* s_cbk, float* s_cbv) {
  const int64_t base = ((int64_t)h * a.n_blk + beta) * a.K * a.G;
  // all 256 byte values get a row (zero past K), so any index byte stays in bounds
  constexpr int CC = C ? C : 1;
  for (int e = threadIdx.x; e < 256 * C; e += blockDim.x) {
    const int r = e / CC, i = e - r * CC;
    const int64_t o = base + (int64_t)r * a.G + i * a.T_c + m;
    s_cbk[e] = r < a.K ? bf16_to_f32(a.kcb[o]) : 0.f;
    s_cbv[e] = r < a.K ? bf16_to_f32(a.vcb[o]) : 0.f;
  }
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

}  // namespace

// fp32 (cos, sin) per (position, frequency): angle p * theta^(-2f/D) in fp64.
__global__ __launch_bounds__(256) void rope_table_f32_kernel(float* tab, int n_pos, int D, double theta) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int H = D / 2;
  if (e >= (int64_t)n_pos * H) return;
  const int p = (int)(e / H), f = (int)(e - (int64_t)p * H);
  const double om = pow(theta, -2.0 * (double)f / (double)D);
  double s, c;
  sincos((double)p * om, &s, &c);
  tab[2 * e] = (float)c;
  tab[2 * e + 1] = (float)s;
}

// Forward on fp32 matrix cores.  Each wave owns 32 queries and computes, per
// tile of 32 keys, S^T = K_rot Q^T (keys on rows, queries on columns: 64
// v_mfma_f32_32x32x2f32 over D) and O^T += V^T P^T (16 steps of two keys x 4
// blocks of 32 channels).  With keys on rows a lane holds 16 of its query's 32
// scores and its partner lane (lane ^ 32) the other 16, so the softmax needs one
// exchange, and the probabilities in the score accumulator are already the B
// operand of the P V product: the key of B row k at step s is the key of
// accumulator register s in half-wave k.  Keys are staged de-interleaved
// ([key][(d % 2) * 64 + d / 2]) so a lane's A operands over D are contiguous;
// values as [key][(d % 32) * 4 + d / 32] so one 16-byte read feeds all four
// channel blocks.
typedef float f32x16_pf __attribute__((ext_vector_type(16)));
constexpr int kMT = 128;              // queries per workgroup (4 waves x 32)

// Keys coded in the pre-transformed space (section 3.3, appendix B eq. 10):
// raw channel d of a key is coordinate p^-1(d) of the rebuilt vector times
// sigma / w[d].  s_pinv[d] = p^-1(d) (identity without a pre-transform; any
// perm input stays in bounds), s_rw[d] = 1 / w[d].  Called by every thread.
__device__ void stage_pretransform(const PrefillArgs& a, int h, int* s_pinv, float* s_rw) {
  for (int e = threadIdx.x; e < kPD; e += blockDim.x) {
    s_pinv[e] = e;
    s_rw[e] = 1.f / a.w[h * kPD + e];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kPD; e += blockDim.x) s_pinv[a.perm[h * kPD + e] & (kPD - 1)] = e;
}

// sigma of token j at step t (pre-transformed keys only)
__device__ __forceinline__ float key_sigma(const PrefillArgs& a, int b, int j, int t) {
  const uint16_t hb = a.sigma[((int64_t)b * a.sig_cap + j) * a.T + t];
  _Float16 hv;
  __builtin_memcpy(&hv, &hb, 2);
  return (float)hv;
}

// Stage cnt keys (rotated) and values for the matrix-core kernels: keys
// de-interleaved into s_k; values block-interleaved into s_v (V_DEINT: like
// the keys instead); s_kb, when given, gets a block-interleaved copy of the keys.
template <int C, bool PT, bool V_DEINT = false>
__device__ void fill_tile_mfma(const PrefillArgs& a, int b, int h, int t, int beta, bool sinks, int j0, int cnt,
                               const float* s_cbk, const float* s_cbv, const int* s_pinv, const float* s_rw,
                               float (*s_k)[kLds], float (*s_v)[kLds], float (*s_kb)[kLds] = nullptr) {
  const int kk = threadIdx.x >> 3, fs = threadIdx.x & 7;
  float klo[8], khi[8], vlo[8], vhi[8];
  if (kk < cnt) {
    const int j = j0 + kk;
    int pos;
    if (sinks) {
      pos = j;
      const int64_t ro = ((((int64_t)b * a.H + h) * a.T + t) * a.n_s + j) * kPD;
      const uint4 xl = *reinterpret_cast<const uint4*>(a.sk + ro + 8 * fs);
      const uint4 xh = *reinterpret_cast<const uint4*>(a.sk + ro + kPH + 8 * fs);
      const uint4 yl = *reinterpret_cast<const uint4*>(a.sv + ro + 8 * fs);
      const uint4 yh = *reinterpret_cast<const uint4*>(a.sv + ro + kPH + 8 * fs);
      const uint32_t wxl[4] = {xl.x, xl.y, xl.z, xl.w}, wxh[4] = {xh.x, xh.y, xh.z, xh.w};
      const uint32_t wyl[4] = {yl.x, yl.y, yl.z, yl.w}, wyh[4] = {yh.x, yh.y, yh.z, yh.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        klo[2 * w] = bf16lo(wxl[w]); klo[2 * w + 1] = bf16hi(wxl[w]);
        khi[2 * w] = bf16lo(wxh[w]); khi[2 * w + 1] = bf16hi(wxh[w]);
        vlo[2 * w] = bf16lo(wyl[w]); vlo[2 * w + 1] = bf16hi(wyl[w]);
        vhi[2 * w] = bf16lo(wyh[w]); vhi[2 * w + 1] = bf16hi(wyh[w]);
      }
    } else if constexpr (C == 0) {
      // precise cache: token j of step t as stored
      pos = a.n_s + j;
      const int64_t ro = ((((int64_t)b * a.H + h) * a.T + t) * a.N_x + j) * kPD;
      const uint4 xl = *reinterpret_cast<const uint4*>(a.xk + ro + 8 * fs);
      const uint4 xh = *reinterpret_cast<const uint4*>(a.xk + ro + kPH + 8 * fs);
      const uint4 yl = *reinterpret_cast<const uint4*>(a.xv + ro + 8 * fs);
      const uint4 yh = *reinterpret_cast<const uint4*>(a.xv + ro + kPH + 8 * fs);
      const uint32_t wxl[4] = {xl.x, xl.y, xl.z, xl.w}, wxh[4] = {xh.x, xh.y, xh.z, xh.w};
      const uint32_t wyl[4] = {yl.x, yl.y, yl.z, yl.w}, wyh[4] = {yh.x, yh.y, yh.z, yh.w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        klo[2 * w] = bf16lo(wxl[w]); klo[2 * w + 1] = bf16hi(wxl[w]);
        khi[2 * w] = bf16lo(wxh[w]); khi[2 * w + 1] = bf16hi(wxh[w]);
        vlo[2 * w] = bf16lo(wyl[w]); vlo[2 * w + 1] = bf16hi(wyl[w]);
        vhi[2 * w] = bf16lo(wyh[w]); vhi[2 * w + 1] = bf16hi(wyh[w]);
      }
    } else {
      pos = a.n_s + j;
      const int64_t ir = ((((int64_t)b * a.H + h) * a.n_blk + beta) * a.N_cap + j) * (kPD / C);
      const uint8_t* kr = a.kidx + ir;
      const uint8_t* vr = a.vidx + ir;
      const float sg = PT ? key_sigma(a, b, j, t) : 1.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int dl = 8 * fs + e, dh = kPH + 8 * fs + e;
        if constexpr (PT) {
          const int zl = s_pinv[dl], zh = s_pinv[dh];
          klo[e] = s_cbk[kr[zl / C] * C + zl % C] * (sg * s_rw[dl]);
          khi[e] = s_cbk[kr[zh / C] * C + zh % C] * (sg * s_rw[dh]);
        } else {
          klo[e] = s_cbk[kr[dl / C] * C + dl % C];
          khi[e] = s_cbk[kr[dh / C] * C + dh % C];
        }
        vlo[e] = s_cbv[vr[dl / C] * C + dl % C];
        vhi[e] = s_cbv[vr[dh / C] * C + dh % C];
      }
    }
    const float4* cs = reinterpret_cast<const float4*>(a.rope + ((int64_t)pos * kPH + 8 * fs) * 2);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2) {
      const float4 w = cs[e2];
      const float a0 = klo[2 * e2], b0 = khi[2 * e2], a1 = klo[2 * e2 + 1], b1 = khi[2 * e2 + 1];
      klo[2 * e2] = a0 * w.x - b0 * w.y;
      khi[2 * e2] = b0 * w.x + a0 * w.y;
      klo[2 * e2 + 1] = a1 * w.z - b1 * w.w;
      khi[2 * e2 + 1] = b1 * w.z + a1 * w.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) klo[e] = khi[e] = vlo[e] = vhi[e] = 0.f;
  }
  // keys: channel d at (d % 2) * 64 + d / 2 (low channels 8fs + e, high 64 + 8fs + e)
  *reinterpret_cast<float4*>(&s_k[kk][4 * fs]) = make_float4(klo[0], klo[2], klo[4], klo[6]);
  *reinterpret_cast<float4*>(&s_k[kk][kPH + 4 * fs]) = make_float4(klo[1], klo[3], klo[5], klo[7]);
  *reinterpret_cast<float4*>(&s_k[kk][32 + 4 * fs]) = make_float4(khi[0], khi[2], khi[4], khi[6]);
  *reinterpret_cast<float4*>(&s_k[kk][kPH + 32 + 4 * fs]) = make_float4(khi[1], khi[3], khi[5], khi[7]);
  if constexpr (V_DEINT) {
    *reinterpret_cast<float4*>(&s_v[kk][4 * fs]) = make_float4(vlo[0], vlo[2], vlo[4], vlo[6]);
    *reinterpret_cast<float4*>(&s_v[kk][kPH + 4 * fs]) = make_float4(vlo[1], vlo[3], vlo[5], vlo[7]);
    *reinterpret_cast<float4*>(&s_v[kk][32 + 4 * fs]) = make_float4(vhi[0], vhi[2], vhi[4], vhi[6]);
    *reinterpret_cast<float4*>(&s_v[kk][kPH + 32 + 4 * fs]) = make_float4(vhi[1], vhi[3], vhi[5], vhi[7]);
  } else {
    // values: channel d at (d % 32) * 4 + d / 32
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dl = 8 * fs + e, dh = kPH + 8 * fs + e;
      s_v[kk][(dl & 31) * 4 + (dl >> 5)] = vlo[e];
      s_v[kk][(dh & 31) * 4 + (dh >> 5)] = vhi[e];
    }
  }
  if (s_kb) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dl = 8 * fs + e, dh = kPH + 8 * fs + e;
      s_kb[kk][(dl & 31) * 4 + (dl >> 5)] = klo[e];
      s_kb[kk][(dh & 31) * 4 + (dh >> 5)] = khi[e];
    }
  }
}

template <int C, bool PT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_fwd_mfma_kernel(PrefillArgs a) {
  extern __shared__ float s_cb[];                    // [2][256*C] step slices
  // two tile buffers: the next tile is staged while the current one is used
  __shared__ __attribute__((aligned(16))) float s_k[2][kTile][kLds];
  __shared__ __attribute__((aligned(16))) float s_v[2][kTile][kLds];
  __shared__ int s_pinv[kPD];
  __shared__ float s_rw[kPD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane >> 5, col = lane & 31;
  const int hq = blockIdx.y, h = hq / a.gqa;
  const int b = blockIdx.z / a.n_steps, tl = blockIdx.z - b * a.n_steps;
  const int t = a.step0 + tl, beta = t / a.T_c, m = t - beta * a.T_c;
  // the last query tiles attend the most tokens: dispatch them first
  const int q0 = (gridDim.x - 1 - blockIdx.x) * kMT;
  const int qw0 = q0 + wave * 32;
  const int i = qw0 + col;
  const bool vq = i < a.N;
  float* s_cbk = s_cb;
  float* s_cbv = s_cb + 256 * C;
  stage_codebooks<C>(a, h, beta, m, s_cbk, s_cbv);
  if constexpr (PT) stage_pretransform(a, h, s_pinv, s_rw);

  // B operand of S^T: qreg[s] = q[i][2s + hh], scaled to base-2 scores
  const int64_t qrow = ((((int64_t)b * a.Hq + hq) * a.n_steps + tl) * a.N + (vq ? i : 0)) * kPD;
  const float qs = vq ? a.scale * kLog2e : 0.f;
  float qreg[64];
  {
    const float4* qp = reinterpret_cast<const float4*>(a.q + qrow);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float4 x = qp[2 * u], y = qp[2 * u + 1];          // channels 8u .. 8u+7
      qreg[4 * u + 0] = (hh ? x.y : x.x) * qs;
      qreg[4 * u + 1] = (hh ? x.w : x.z) * qs;
      qreg[4 * u + 2] = (hh ? y.y : y.x) * qs;
      qreg[4 * u + 3] = (hh ? y.w : y.z) * qs;
    }
  }
  f32x16_pf o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float mx = -INFINITY, l = 0.f;

  auto consume = [&](int cnt, int j0, bool sinks, int buf) {
    if (!sinks && qw0 + 31 < j0) return;             // every query of the wave precedes the tile
    f32x16_pf sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 16; ++s4) {
      const float4 kv = *reinterpret_cast<const float4*>(&s_k[buf][col][hh * kPH + 4 * s4]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.x, qreg[4 * s4 + 0], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.y, qreg[4 * s4 + 1], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.z, qreg[4 * s4 + 2], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.w, qreg[4 * s4 + 3], sacc, 0, 0, 0);
    }
    // register r holds key j0 + 8(r/4) + 4hh + r%4 of query i
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 8 * (r >> 2) + 4 * hh + (r & 3);
      const bool ok = vq && kr < cnt && (sinks || j0 + kr <= i);
      sacc[r] = ok ? sacc[r] : -INFINITY;
      tmax = fmaxf(tmax, sacc[r]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mn = fmaxf(mx, tmax);
    const float al = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mx - mn);
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sacc[r] = sacc[r] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sacc[r] - mn);
      ps += sacc[r];
    }
    ps += __shfl_xor(ps, 32);
    l = l * al + ps;
    mx = mn;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= al;
    // O^T += V^T P^T: at step s, B row hh is this lane's register s
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int kr = 8 * (st >> 2) + 4 * hh + (st & 3);
      const float4 vv = *reinterpret_cast<const float4*>(&s_v[buf][kr][col * 4]);
      o[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.x, sacc[st], o[0], 0, 0, 0);
      o[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.y, sacc[st], o[1], 0, 0, 0);
      o[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.z, sacc[st], o[2], 0, 0, 0);
      o[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.w, sacc[st], o[3], 0, 0, 0);
    }
  };
  // tiles: the sinks first, then the tokens up to this workgroup's last query
  const int jend = min(a.N, q0 + kMT);
  const int ns_t = (a.n_s + kTile - 1) / kTile, ntl = ns_t + (jend + kTile - 1) / kTile;
  auto info = [&](int k, bool& sinks, int& j0, int& cnt) {
    sinks = k < ns_t;
    j0 = kTile * (sinks ? k : k - ns_t);
    cnt = min(kTile, (sinks ? a.n_s : jend) - j0);
  };
  __syncthreads();                                   // codebook slices staged
  if (ntl > 0) {
    bool sk;
    int j0, cnt;
    info(0, sk, j0, cnt);
    fill_tile_mfma<C, PT>(a, b, h, t, beta, sk, j0, cnt, s_cbk, s_cbv, s_pinv, s_rw, s_k[0], s_v[0]);
  }
  __syncthreads();
  for (int k = 0; k < ntl; ++k) {
    bool sk;
    int j0, cnt;
    if (k + 1 < ntl) {
      info(k + 1, sk, j0, cnt);
      fill_tile_mfma<C, PT>(a, b, h, t, beta, sk, j0, cnt, s_cbk, s_cbv, s_pinv, s_rw, s_k[(k + 1) & 1], s_v[(k + 1) & 1]);
    }
    info(k, sk, j0, cnt);
    consume(cnt, j0, sk, k & 1);
    __syncthreads();                                 // tile k+1 staged, tile k no longer read
  }
  if (vq) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* op = a.out + qrow;
    // O^T register r of block db is channel 32db + 8(r/4) + 4hh + r%4
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(op + 32 * db + 8 * r4 + 4 * hh) =
            make_float4(o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv, o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
    if (hh == 0) a.lse[qrow / kPD] = l > 0.f ? (mx + __log2f(l)) * kLn2 : -INFINITY;
  }
}

// Query-side backward on fp32 matrix cores (layout as the forward): per tile
// of 32 keys, S^T = K_rot Q^T and dP^T = V dO^T (keys on rows), dS^T = P^T
// (dP^T - delta) with P^T = exp(S^T - lse), and dQ^T += K_rot^T dS^T, whose B
// operand is the dS^T accumulator itself.
template <int C, bool PT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_bwd_q_mfma_kernel(
    PrefillArgs a) {
  extern __shared__ float s_cb[];
  __shared__ __attribute__((aligned(16))) float s_k[kTile][kLds];
  __shared__ __attribute__((aligned(16))) float s_v[kTile][kLds];
  __shared__ __attribute__((aligned(16))) float s_kb[kTile][kLds];
  __shared__ int s_pinv[kPD];
  __shared__ float s_rw[kPD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane >> 5, col = lane & 31;
  const int hq = blockIdx.y, h = hq / a.gqa;
  const int b = blockIdx.z / a.n_steps, tl = blockIdx.z - b * a.n_steps;
  const int t = a.step0 + tl, beta = t / a.T_c, m = t - beta * a.T_c;
  const int q0 = (gridDim.x - 1 - blockIdx.x) * kMT;
  const int qw0 = q0 + wave * 32;
  const int i = qw0 + col;
  const bool vq = i < a.N;
  float* s_cbk = s_cb;
  float* s_cbv = s_cb + 256 * C;
  stage_codebooks<C>(a, h, beta, m, s_cbk, s_cbv);
  if constexpr (PT) stage_pretransform(a, h, s_pinv, s_rw);

  const int64_t qr = (((int64_t)b * a.Hq + hq) * a.n_steps + tl) * a.N + (vq ? i : 0);
  const float qs = vq ? a.scale * kLog2e : 0.f;
  float qreg[64], dreg[64];
  {
    const float4* qp = reinterpret_cast<const float4*>(a.q + qr * kPD);
    const float4* dp = reinterpret_cast<const float4*>(a.dout + qr * kPD);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const float4 x = qp[2 * u], y = qp[2 * u + 1];
      qreg[4 * u + 0] = (hh ? x.y : x.x) * qs;
      qreg[4 * u + 1] = (hh ? x.w : x.z) * qs;
      qreg[4 * u + 2] = (hh ? y.y : y.x) * qs;
      qreg[4 * u + 3] = (hh ? y.w : y.z) * qs;
      const float4 x2 = dp[2 * u], y2 = dp[2 * u + 1];
      const float dsc = vq ? 1.f : 0.f;
      dreg[4 * u + 0] = (hh ? x2.y : x2.x) * dsc;
      dreg[4 * u + 1] = (hh ? x2.w : x2.z) * dsc;
      dreg[4 * u + 2] = (hh ? y2.y : y2.x) * dsc;
      dreg[4 * u + 3] = (hh ? y2.w : y2.z) * dsc;
    }
  }
  const float l2 = a.lse[qr] * kLog2e, dl = a.delta[qr];
  f32x16_pf dq[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[db][r] = 0.f;

  auto consume = [&](int cnt, int j0, bool sinks) {
    if (!sinks && qw0 + 31 < j0) return;
    f32x16_pf sacc, pacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 16; ++s4) {
      const float4 kv = *reinterpret_cast<const float4*>(&s_k[col][hh * kPH + 4 * s4]);
      const float4 vv = *reinterpret_cast<const float4*>(&s_v[col][hh * kPH + 4 * s4]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.x, qreg[4 * s4 + 0], sacc, 0, 0, 0);
      pacc = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.x, dreg[4 * s4 + 0], pacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.y, qreg[4 * s4 + 1], sacc, 0, 0, 0);
      pacc = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.y, dreg[4 * s4 + 1], pacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.z, qreg[4 * s4 + 2], sacc, 0, 0, 0);
      pacc = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.z, dreg[4 * s4 + 2], pacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kv.w, qreg[4 * s4 + 3], sacc, 0, 0, 0);
      pacc = __builtin_amdgcn_mfma_f32_32x32x2f32(vv.w, dreg[4 * s4 + 3], pacc, 0, 0, 0);
    }
    // dS^T in place of the score accumulator (masked pairs contribute zero)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 8 * (r >> 2) + 4 * hh + (r & 3);
      const bool ok = vq && kr < cnt && (sinks || j0 + kr <= i);
      const float p = ok ? __builtin_amdgcn_exp2f(sacc[r] - l2) : 0.f;
      sacc[r] = p * (pacc[r] - dl);
    }
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int kr = 8 * (st >> 2) + 4 * hh + (st & 3);
      const float4 kb = *reinterpret_cast<const float4*>(&s_kb[kr][col * 4]);
      dq[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(kb.x, sacc[st], dq[0], 0, 0, 0);
      dq[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(kb.y, sacc[st], dq[1], 0, 0, 0);
      dq[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(kb.z, sacc[st], dq[2], 0, 0, 0);
      dq[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(kb.w, sacc[st], dq[3], 0, 0, 0);
    }
  };
  for (int j0 = 0; j0 < a.n_s; j0 += kTile) {
    const int cnt = min(kTile, a.n_s - j0);
    __syncthreads();
    fill_tile_mfma<C, PT, true>(a, b, h, t, beta, true, j0, cnt, s_cbk, s_cbv, s_pinv, s_rw, s_k, s_v, s_kb);
    __syncthreads();
    consume(cnt, j0, true);
  }
  const int jend = min(a.N, q0 + kMT);
  for (int j0 = 0; j0 < jend; j0 += kTile) {
    const int cnt = min(kTile, jend - j0);
    __syncthreads();
    fill_tile_mfma<C, PT, true>(a, b, h, t, beta, false, j0, cnt, s_cbk, s_cbv, s_pinv, s_rw, s_k, s_v, s_kb);
    __syncthreads();
    consume(cnt, j0, false);
  }
  if (vq) {
    float* op = a.dq + qr * kPD;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<float4*>(op + 32 * db + 8 * r4 + 4 * hh) =
            make_float4(dq[db][4 * r4] * a.scale, dq[db][4 * r4 + 1] * a.scale, dq[db][4 * r4 + 2] * a.scale,
                        dq[db][4 * r4 + 3] * a.scale);
  }
}

// Key-side backward on fp32 matrix cores, in two passes so that each fits the
// register file.  A workgroup owns 128 tokens (32 per wave, one per lane
// column) and walks the tiles of 32 queries that can see them.  With the
// queries on rows, S = Q K_rot^T has each lane's token in its column, so the
// token's own rotated key (and value) are the B operands, kept in registers
// as channels 2s + hh, and the probabilities in the accumulator are the B
// operand of the next product:
//   V pass: dV^T += dO^T P;
//   K pass: dP = dO V^T, dS = P (dP - delta), dK_rot^T += Q^T dS.
// Query tiles are staged de-interleaved ([q][(d % 2) * 64 + d / 2]) for the A
// operands over D and block-interleaved ([q][(d % 32) * 4 + d / 32]) for the A
// operands over the query pairs.  The gradients are added per codeword in LDS,
// then into the global fp32 gradient.

// Stage tile rows of queries (and dO): thread (r, part) writes channels
// 16 part .. 16 part + 15 of row r.
__device__ __forceinline__ void stage_rows(const float* src, float sc, float (*deint)[kLds], float (*blk)[kLds],
                                           int r, int part) {
  const float4* p4 = reinterpret_cast<const float4*>(src + 16 * part);
  float x[16];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float4 v = p4[u];
    x[4 * u] = v.x * sc; x[4 * u + 1] = v.y * sc; x[4 * u + 2] = v.z * sc; x[4 * u + 3] = v.w * sc;
  }
  if (deint) {
    *reinterpret_cast<float4*>(&deint[r][8 * part]) = make_float4(x[0], x[2], x[4], x[6]);
    *reinterpret_cast<float4*>(&deint[r][8 * part + 4]) = make_float4(x[8], x[10], x[12], x[14]);
    *reinterpret_cast<float4*>(&deint[r][kPH + 8 * part]) = make_float4(x[1], x[3], x[5], x[7]);
    *reinterpret_cast<float4*>(&deint[r][kPH + 8 * part + 4]) = make_float4(x[9], x[11], x[13], x[15]);
  }
  if (blk) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int d = 16 * part + e;
      blk[r][(d & 31) * 4 + (d >> 5)] = x[e];
    }
  }
}

// This lane's token: rotated key channels kreg[s] = k_rot[2s + hh] and value
// channels vreg[s] = v[2s + hh] (s < 64), from the codebooks.
template <int C, bool PT, bool WITH_V>
__device__ __forceinline__ void token_regs(const PrefillArgs& a, int64_t ir, int64_t cbo, int m, int pos, int hh,
                                           float sg, const int* s_pinv, const float* s_rw, float (&kreg)[64],
                                           float (&vreg)[64]) {
  const float2* rp = reinterpret_cast<const float2*>(a.rope + (int64_t)pos * kPH * 2);
  if constexpr (C == 0) {
    // precise cache: ir is the row offset of the token's key and value
#pragma unroll
    for (int s = 0; s < 32; ++s) {
      const int dl = 2 * s + hh, dh = dl + kPH;
      const float xl = bf16_to_f32(a.xk[ir + dl]), xh = bf16_to_f32(a.xk[ir + dh]);
      const float2 w = rp[dl];
      kreg[s] = xl * w.x - xh * w.y;
      kreg[s + 32] = xh * w.x + xl * w.y;
      if constexpr (WITH_V) {
        vreg[s] = bf16_to_f32(a.xv[ir + dl]);
        vreg[s + 32] = bf16_to_f32(a.xv[ir + dh]);
      }
    }
    return;
  }
  constexpr int CC = C ? C : 1;
#pragma unroll
  for (int s = 0; s < 32; ++s) {
    const int dl = 2 * s + hh, dh = dl + kPH;
    const int zl = PT ? s_pinv[dl] : dl, zh = PT ? s_pinv[dh] : dh;
    const float fl = PT ? sg * s_rw[dl] : 1.f, fh = PT ? sg * s_rw[dh] : 1.f;
    // an index byte >= K (never written by the encode) reads the last entry
    const int rl = min((int)a.kidx[ir + zl / CC], a.K - 1), rh = min((int)a.kidx[ir + zh / CC], a.K - 1);
    const float xl = bf16_to_f32(a.kcb[cbo + (int64_t)rl * a.G + (zl % CC) * a.T_c + m]) * fl;
    const float xh = bf16_to_f32(a.kcb[cbo + (int64_t)rh * a.G + (zh % CC) * a.T_c + m]) * fh;
    const float2 w = rp[dl];
    kreg[s] = xl * w.x - xh * w.y;
    kreg[s + 32] = xh * w.x + xl * w.y;
    if constexpr (WITH_V) {
      const int ul = min((int)a.vidx[ir + dl / CC], a.K - 1), uh = min((int)a.vidx[ir + dh / CC], a.K - 1);
      vreg[s] = bf16_to_f32(a.vcb[cbo + (int64_t)ul * a.G + (dl % CC) * a.T_c + m]);
      vreg[s + 32] = bf16_to_f32(a.vcb[cbo + (int64_t)uh * a.G + (dh % CC) * a.T_c + m]);
    }
  }
}

template <int C, bool PT, bool KPASS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void prefill_bwd_kv_mfma_kernel(
    PrefillArgs a) {
  extern __shared__ float s_g[];                      // [256][C] gradient of this step's slice
  __shared__ __attribute__((aligned(16))) float s_q[kTile][kLds];      // q, de-interleaved, base-2 scaled
  __shared__ __attribute__((aligned(16))) float s_b[kTile][kLds];      // V pass: dO blocks; K pass: q blocks
  __shared__ __attribute__((aligned(16))) float s_d[KPASS ? kTile : 1][kLds];   // K pass: dO, de-interleaved
  __shared__ float s_l2[kTile], s_dl[kTile];
  __shared__ int s_pinv[kPD];
  __shared__ float s_rw[kPD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hh = lane >> 5, col = lane & 31;
  const int hq = blockIdx.y, h = hq / a.gqa;
  const int b = blockIdx.z / a.n_steps, tl = blockIdx.z - b * a.n_steps;
  const int t = a.step0 + tl, beta = t / a.T_c, m = t - beta * a.T_c;
  const int k0 = blockIdx.x * kMT;
  const int kw0 = k0 + 32 * wave;
  const int j = kw0 + col;
  const bool vk = j < a.N;
  for (int e = threadIdx.x; e < 256 * C; e += blockDim.x) s_g[e] = 0.f;
  if constexpr (PT) stage_pretransform(a, h, s_pinv, s_rw);
  __syncthreads();

  constexpr int CC = C ? C : 1;
  // index row of the token (precise cache: row offset of its key and value)
  const int64_t ir = C ? ((((int64_t)b * a.H + h) * a.n_blk + beta) * a.N_cap + (vk ? j : 0)) * (kPD / CC)
                       : ((((int64_t)b * a.H + h) * a.T + t) * a.N_x + (vk ? j : 0)) * kPD;
  const int64_t cbo = ((int64_t)h * a.n_blk + beta) * a.K * a.G;
  const int pos = a.n_s + (vk ? j : 0);
  const float sg = PT ? key_sigma(a, b, vk ? j : 0, t) : 1.f;
  float kreg[64], vreg[64];
  token_regs<C, PT, KPASS>(a, ir, cbo, m, pos, hh, sg, s_pinv, s_rw, kreg, vreg);
  f32x16_pf acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;
  const float sc2 = a.scale * kLog2e;
  const int64_t row0 = (((int64_t)b * a.Hq + hq) * a.n_steps + tl) * a.N;

  for (int i0 = k0; i0 < a.N; i0 += kTile) {
    const int cnt = min(kTile, a.N - i0);
    __syncthreads();
    {
      const int r = threadIdx.x >> 3, part = threadIdx.x & 7;
      if (r < cnt) {
        const int64_t qr = row0 + i0 + r;
        stage_rows(a.q + qr * kPD, sc2, s_q, nullptr, r, part);
        if constexpr (KPASS) {
          stage_rows(a.q + qr * kPD, 1.f, nullptr, s_b, r, part);
          stage_rows(a.dout + qr * kPD, 1.f, s_d, nullptr, r, part);
        } else {
          stage_rows(a.dout + qr * kPD, 1.f, nullptr, s_b, r, part);
        }
        if (part == 0) {
          s_l2[r] = a.lse[qr] * kLog2e;
          s_dl[r] = a.delta[qr];
        }
      } else {
        // rows past the end: zero operands
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          s_q[r][16 * part + e] = 0.f;
          s_b[r][16 * part + e] = 0.f;
          if constexpr (KPASS) s_d[r][16 * part + e] = 0.f;
        }
        if (part == 0) s_l2[r] = s_dl[r] = 0.f;
      }
    }
    __syncthreads();
    if (i0 + kTile - 1 < kw0) continue;              // these queries see none of the wave's tokens
    f32x16_pf sacc, pacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.f;
#pragma unroll
    for (int s4 = 0; s4 < 16; ++s4) {
      const float4 qv = *reinterpret_cast<const float4*>(&s_q[col][hh * kPH + 4 * s4]);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.x, kreg[4 * s4 + 0], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.y, kreg[4 * s4 + 1], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.z, kreg[4 * s4 + 2], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(qv.w, kreg[4 * s4 + 3], sacc, 0, 0, 0);
      if constexpr (KPASS) {
        const float4 dv = *reinterpret_cast<const float4*>(&s_d[col][hh * kPH + 4 * s4]);
        pacc = __builtin_amdgcn_mfma_f32_32x32x2f32(dv.x, vreg[4 * s4 + 0], pacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x2f32(dv.y, vreg[4 * s4 + 1], pacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x2f32(dv.z, vreg[4 * s4 + 2], pacc, 0, 0, 0);
        pacc = __builtin_amdgcn_mfma_f32_32x32x2f32(dv.w, vreg[4 * s4 + 3], pacc, 0, 0, 0);
      }
    }
    // register r: query i0 + 8(r/4) + 4hh + r%4 of this lane's token j
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qrl = 8 * (r >> 2) + 4 * hh + (r & 3);
      const bool ok = vk && qrl < cnt && j <= i0 + qrl;
      const float p = ok ? __builtin_amdgcn_exp2f(sacc[r] - s_l2[qrl]) : 0.f;
      if constexpr (KPASS)
        sacc[r] = p * (pacc[r] - s_dl[qrl]);
      else
        sacc[r] = p;
    }
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int qrl = 8 * (st >> 2) + 4 * hh + (st & 3);
      const float4 bb = *reinterpret_cast<const float4*>(&s_b[qrl][col * 4]);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(bb.x, sacc[st], acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(bb.y, sacc[st], acc[1], 0, 0, 0);
      acc[2] = __builtin_amdgcn_mfma_f32_32x32x2f32(bb.z, sacc[st], acc[2], 0, 0, 0);
      acc[3] = __builtin_amdgcn_mfma_f32_32x32x2f32(bb.w, sacc[st], acc[3], 0, 0, 0);
    }
  }
  // acc[db][r] is the gradient of channel 32db + 8(r/4) + 4hh + r%4 of token j
  // (K pass: of its rotated key, before the 1/sqrt(D) scale)
  if (vk && C == 0) {
    // precise cache: the gradient of this token's pre-RoPE key (rotation
    // undone) or value, added (q-heads of a GQA group share the token)
    if constexpr (KPASS) {
      const float2* rp = reinterpret_cast<const float2*>(a.rope + (int64_t)pos * kPH * 2);
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dl = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3), dh = dl + kPH;
          const float2 w = rp[dl];
          unsafeAtomicAdd(&a.dxk[ir + dl], (acc[db][r] * w.x + acc[db + 2][r] * w.y) * a.scale);
          unsafeAtomicAdd(&a.dxk[ir + dh], (acc[db + 2][r] * w.x - acc[db][r] * w.y) * a.scale);
        }
    } else {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) unsafeAtomicAdd(&a.dxv[ir + 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3)], acc[db][r]);
    }
  } else if (vk) {
    if constexpr (KPASS) {
      const float2* rp = reinterpret_cast<const float2*>(a.rope + (int64_t)pos * kPH * 2);
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dl = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3), dh = dl + kPH;
          const float2 w = rp[dl];
          // undo the rotation, then the pre-transform's scale; raw channel d
          // came from coordinate p^-1(d) of the rebuilt vector
          const float gl = (acc[db][r] * w.x + acc[db + 2][r] * w.y) * (PT ? a.scale * sg * s_rw[dl] : a.scale);
          const float gh = (acc[db + 2][r] * w.x - acc[db][r] * w.y) * (PT ? a.scale * sg * s_rw[dh] : a.scale);
          const int zl = PT ? s_pinv[dl] : dl, zh = PT ? s_pinv[dh] : dh;
          atomicAdd(&s_g[a.kidx[ir + zl / CC] * C + zl % CC], gl);
          atomicAdd(&s_g[a.kidx[ir + zh / CC] * C + zh % CC], gh);
        }
    } else {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = 32 * db + 8 * (r >> 2) + 4 * hh + (r & 3);
          atomicAdd(&s_g[a.vidx[ir + d / CC] * C + d % CC], acc[db][r]);
        }
    }
  }
  __syncthreads();
  float* g = KPASS ? a.dkcb : a.dvcb;
  for (int e = threadIdx.x; e < a.K * C; e += blockDim.x) {
    const int r = e / CC, i = e - r * CC;
    if (s_g[e] != 0.f) unsafeAtomicAdd(&g[cbo + (int64_t)r * a.G + i * a.T_c + m], s_g[e]);
  }
}

// delta[row] = sum_d dout[row][d] * out[row][d]; one wave per row.
__global__ __launch_bounds__(256) void prefill_delta_kernel(const float* __restrict__ out,
                                                            const float* __restrict__ dout,
                                                            float* __restrict__ delta, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const float2 x = reinterpret_cast<const float2*>(out + r * kPD)[lane];
  const float2 y = reinterpret_cast<const float2*>(dout + r * kPD)[lane];
  float s = x.x * y.x + x.y * y.y;
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) delta[r] = s;
}

__global__ __launch_bounds__(256) void prefill_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n) p[e] = 0.f;
}

hipError_t launch_fill_f32(float* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_rope_table_f32(float* tab, int n_pos, int D, double theta, hipStream_t s) {
  const int64_t n = (int64_t)n_pos * (D / 2);
  hipLaunchKernelGGL(rope_table_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tab, n_pos, D, theta);
  return hipGetLastError();
}

template <int C, bool PT>
static hipError_t prefill_launch(const PrefillArgs& a, bool backward, hipStream_t s) {
  const size_t lds = (size_t)2 * 256 * C * sizeof(float);
  // dynamic LDS beyond the default allowance (C = 32 takes 64 KiB; the
  // precise cache, C = 0, none)
  for (const void* k : {reinterpret_cast<const void*>(&prefill_fwd_mfma_kernel<C, PT>),
                        reinterpret_cast<const void*>(&prefill_bwd_kv_mfma_kernel<C, PT, false>),
                        reinterpret_cast<const void*>(&prefill_bwd_kv_mfma_kernel<C, PT, true>),
                        reinterpret_cast<const void*>(&prefill_bwd_q_mfma_kernel<C, PT>)}) {
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (!backward) {
    const dim3 gm((a.N + kMT - 1) / kMT, a.Hq, a.B * a.n_steps);
    hipLaunchKernelGGL((prefill_fwd_mfma_kernel<C, PT>), gm, dim3(256), lds, s, a);
    return hipGetLastError();
  }
  const int64_t rows = (int64_t)a.B * a.Hq * a.n_steps * a.N;
  hipLaunchKernelGGL(prefill_delta_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, a.out, a.dout,
                     a.delta, rows);
  if constexpr (C != 0) {
    const int64_t ncb = (int64_t)a.H * a.n_blk * a.K * a.G;
    hipLaunchKernelGGL(prefill_zero_kernel, dim3((unsigned)((ncb + 255) / 256)), dim3(256), 0, s, a.dkcb, ncb);
    hipLaunchKernelGGL(prefill_zero_kernel, dim3((unsigned)((ncb + 255) / 256)), dim3(256), 0, s, a.dvcb, ncb);
  }
  const dim3 gk((a.N + kMT - 1) / kMT, a.Hq, a.B * a.n_steps);
  const size_t lds_g = (size_t)256 * C * sizeof(float);
  hipLaunchKernelGGL((prefill_bwd_kv_mfma_kernel<C, PT, false>), gk, dim3(256), lds_g, s, a);
  hipLaunchKernelGGL((prefill_bwd_kv_mfma_kernel<C, PT, true>), gk, dim3(256), lds_g, s, a);
  const dim3 gm((a.N + kMT - 1) / kMT, a.Hq, a.B * a.n_steps);
  hipLaunchKernelGGL((prefill_bwd_q_mfma_kernel<C, PT>), gm, dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int C>
static hipError_t prefill_launch_pt(const PrefillArgs& a, bool backward, hipStream_t s) {
  return a.perm ? prefill_launch<C, true>(a, backward, s) : prefill_launch<C, false>(a, backward, s);
}

hipError_t launch_prefill(const PrefillArgs& a, int C, bool backward, hipStream_t s) {
  switch (C) {
    case 0: return prefill_launch<0, false>(a, backward, s);
    case 2: return prefill_launch_pt<2>(a, backward, s);
    case 4: return prefill_launch_pt<4>(a, backward, s);
    case 8: return prefill_launch_pt<8>(a, backward, s);
    case 16: return prefill_launch_pt<16>(a, backward, s);
    case 32: return prefill_launch_pt<32>(a, backward, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace loopvq
