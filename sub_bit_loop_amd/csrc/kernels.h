// Kernel argument blocks and launchers shared by the LoopVQ host API and the
// HIP kernels.  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loopvq {

struct EncodeArgs {
  const uint16_t* x;          // bf16 rows of D, strides in elements
  int64_t xs0, xs1, xs2, xs3;
  const uint16_t* cb;         // bf16 [H][n_blk][K][G]
  uint8_t* idx;               // [B][H][n_blk][N_cap][D/c]
  int32_t H, n_blk, K, T, N, tok0, N_cap;
  const float* w;             // pre-transform (keys) or null
  const int16_t* perm;
  const uint16_t* sigma;      // fp16 [B][sig_cap][T]
  int32_t sig_cap;
};

struct SigmaArgs {
  const uint16_t* x;
  int64_t xs0, xs1, xs2, xs3;
  int32_t H, T, N, tok0, sig_cap;
  uint16_t* sigma;            // fp16 [B][sig_cap][T]
};

struct DecodeArgs {
  const uint16_t* q;          // bf16 [B][Hq][n_steps][D]
  const uint8_t* kidx;        // [B][H][n_blk][N_cap][D/c]
  const uint8_t* vidx;
  const uint16_t* kcb;        // bf16 [H][n_blk][K][G]
  const uint16_t* vcb;
  const uint16_t* sk;         // bf16 [B][H][T][n_s][D]
  const uint16_t* sv;
  const uint16_t* rk;         // bf16 [B][H][T][r_cap][D] recent window or null
  const uint16_t* rv;
  int32_t n_r, r_cap;
  const int32_t* seq_len;     // [B] or null
  const float* w;             // pre-transform or null
  const int16_t* perm;
  const uint16_t* sigma;      // fp16 [B][sig_cap][T]
  int32_t sig_cap;
  const void* rope;           // fp16 [n_pos][D/8][8] quads (cos x4, sin x4)
  float* ws;                  // partials [B][Hq][n_steps][n_split][D+1]
  int32_t B, H, Hq, T, n_blk, K, N, N_cap, n_s, step0, n_steps, n_split, gqa, blk0, n_blk_serv;
  int32_t tok_per_split;
  float qscale;               // log2(e) / sqrt(D)
  float theta;                // RoPE base the table was made with
  int32_t n_pos;              // positions in the RoPE table
  // One context split (pre-transform, GQA and c = 4 multi-step kernels):
  // with out set, a workgroup writes its rows of out / lse itself and no
  // merge kernel runs (the merge of a single partial returns it unchanged).
  // Several splits always go through merge_kernel: a merge inside the kernel
  // needs device-scope fences (an L2 write-back and invalidate per
  // workgroup), which cost more than the merge launch.
  float* out;                 // fp32 [B][Hq][n_steps][D] or null (partials)
  float* lse;                 // fp32 [B][Hq][n_steps] or null
};

// Largest |value| a decode workgroup converts to fp16 besides its codebooks:
// the queries of q-heads [hq0, hq0 + nh) at steps [t_lo, t_hi) (mq; when kw
// is given, channel d counts divided by min(kw[d], kw[d ^ D/2])) and, for
// the split that attends them (with_bf16), the bf16 sink and recent-window
// keys (mk; channel d multiplied by kw[d] when kw is given) and values (mv)
// of kv-head h at those steps.  Each thread of the workgroup scans a strided
// share of 16-byte chunks; the caller reduces across the workgroup.  The kernels turn these
// into power-of-two range scales (folded back into the scores and outputs),
// so any finite input stays finite in fp16.
__device__ inline void decode_input_absmax(const DecodeArgs& a, int b, int hq0, int nh, int h, int t_lo, int t_hi,
                                           bool with_bf16, const float* kw, float& mq, float& mk, float& mv) {
  constexpr int D = 128, CH = D / 8;   // 16-byte chunks per row (rows are 16-byte aligned)
  const int ns = t_hi - t_lo;
  mq = mk = mv = 0.f;
  if (ns <= 0) return;
  // largest |x| (times the channel factor f(d) when given) over the 8 bf16 of
  // a 16-byte chunk whose first channel is d0
  auto chunk_max = [&](const uint16_t* p, int d0, auto f) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    float m = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m = fmaxf(m, fabsf(__uint_as_float(ws[k] << 16)) * f(d0 + 2 * k));
      m = fmaxf(m, fabsf(__uint_as_float(ws[k] & 0xffff0000u)) * f(d0 + 2 * k + 1));
    }
    return m;
  };
  auto one = [](int) { return 1.f; };
  // queries: rows (q-head hh, step tl)
  for (int e = threadIdx.x; e < nh * ns * CH; e += blockDim.x) {
    const int r = e / CH, c = e - r * CH, hh = r / ns, tl = r - hh * ns;
    const uint16_t* row = a.q + (((int64_t)b * a.Hq + hq0 + hh) * a.n_steps + (t_lo + tl - a.step0)) * D;
    if (kw)
      mq = fmaxf(mq, chunk_max(row + 8 * c, 8 * c, [&](int d) { return 1.f / fminf(kw[d], kw[d ^ (D / 2)]); }));
    else
      mq = fmaxf(mq, chunk_max(row + 8 * c, 8 * c, one));
  }
  if (!with_bf16) return;
  // sinks: the rows of steps t_lo .. t_hi-1 are contiguous
  const int64_t s0 = (((int64_t)b * a.H + h) * a.T + t_lo) * a.n_s * D;
  for (int e = threadIdx.x; e < ns * a.n_s * CH; e += blockDim.x) {
    const int c = e % CH;
    if (kw)
      mk = fmaxf(mk, chunk_max(a.sk + s0 + (int64_t)e * 8, 8 * c, [&](int d) { return kw[d]; }));
    else
      mk = fmaxf(mk, chunk_max(a.sk + s0 + (int64_t)e * 8, 8 * c, one));
    mv = fmaxf(mv, chunk_max(a.sv + s0 + (int64_t)e * 8, 8 * c, one));
  }
  // recent window: rows (step tl, token s < n_r) of capacity r_cap
  for (int e = threadIdx.x; e < ns * a.n_r * CH; e += blockDim.x) {
    const int r = e / CH, c = e - r * CH, tl = r / a.n_r, sr = r - tl * a.n_r;
    const int64_t o = ((((int64_t)b * a.H + h) * a.T + t_lo + tl) * a.r_cap + sr) * D + 8 * c;
    if (kw)
      mk = fmaxf(mk, chunk_max(a.rk + o, 8 * c, [&](int d) { return kw[d]; }));
    else
      mk = fmaxf(mk, chunk_max(a.rk + o, 8 * c, one));
    mv = fmaxf(mv, chunk_max(a.rv + o, 8 * c, one));
  }
}

// Power-of-two range scale of the fp16 decode kernels: the shift s with
// 2^-s * m in [2^(lim-1), 2^lim) for the largest magnitude m of a set of
// values (down or up, up by at most 2^64; 0 for m = 0).  The values enter
// fp16 times 2^-s and 2^s is folded back into the fp32 scores or outputs.
__device__ inline int pow2_range_shift(float m, int lim) {
  if (!(m > 0.f)) return 0;
  return max(ilogbf(m) + 1 - lim, -64);
}

struct TasqStatsArgs {
  const uint16_t* x;          // bf16 rows of D (raw pre-RoPE keys), strides in elements
  int64_t xs0, xs1, xs2, xs3;
  const float* w;             // [H][D]
  const uint16_t* sigma;      // fp16 [B][sig_cap][T]
  int32_t sig_cap;
  double* mean;               // [H][n_blk][T_c*D]
  double* cov;                // [H][n_blk][T_c*D][T_c*D]
  int32_t B, H, T, T_c, n_blk, N, D;
};

struct KmeansArgs {
  const uint16_t* x;          // bf16 rows of D (the encoded K or V cache), strides in elements
  int64_t xs0, xs1, xs2, xs3;
  const uint8_t* idx;         // [B][H][n_blk][N_cap][D/c] assignments (loopvq_encode)
  const float* weight;        // [B][H][n_blk][N][D/c] importance per joint vector, or null (all 1)
  const float* w;             // pre-transform (keys) or null
  const int16_t* perm;
  const uint16_t* sigma;      // fp16 [B][sig_cap][T]
  int32_t sig_cap;
  double* sums;               // [H][n_blk][K][G], accumulated
  double* wsum;               // [H][n_blk][K], accumulated
  int32_t H, T, T_c, n_blk, K, G, N, N_cap, D;
};

struct PrefillArgs {
  const float* q;             // fp32 [B][Hq][n_steps][N][D], post-RoPE
  const uint8_t* kidx;        // [B][H][n_blk][N_cap][D/c]
  const uint8_t* vidx;
  const uint16_t* kcb;        // bf16 [H][n_blk][K][G]
  const uint16_t* vcb;
  const uint16_t* sk;         // bf16 [B][H][T][n_s][D], pre-RoPE
  const uint16_t* sv;
  const float* rope;          // fp32 [n_pos][D/2][2] (cos, sin)
  float* out;                 // fp32 [B][Hq][n_steps][N][D] (written forward, read backward)
  float* lse;                 // fp32 [B][Hq][n_steps][N], natural log
  const float* dout;          // backward: gradient of out
  float* dq;                  // backward: fp32 like q
  float* dkcb;                // backward: fp32 [H][n_blk][K][G]
  float* dvcb;
  float* delta;               // backward scratch: [B][Hq][n_steps][N]
  const float* w;             // keys' pre-transform (or null): w [H][D], perm [H][D],
  const int16_t* perm;        //   sigma fp16 [B][sig_cap][T]
  const uint16_t* sigma;
  int32_t sig_cap;
  int32_t B, H, Hq, T, T_c, n_blk, K, G, N, N_cap, n_s, step0, n_steps, gqa;
  float scale;                // 1 / sqrt(D)
  // precise cache (C = 0): bf16 keys and values [B][H][T][N_x][D], pre-RoPE,
  // and the fp32 gradients added into dxk (pre-RoPE keys) and dxv, same layout
  const uint16_t* xk;
  const uint16_t* xv;
  int32_t N_x;
  float* dxk;
  float* dxv;
};

struct MergeArgs {
  const float* ws;
  float* out;
  float* lse;
  int32_t rows, n_split;
};

// Launchers return hipSuccess or the launch error.  G in {16, 32},
// T_c in {1, 2, 4, 8}; the caller validates.
hipError_t launch_encode(int G, int TC, bool tasq, const EncodeArgs& a, int B, hipStream_t s);
hipError_t launch_sigma(const SigmaArgs& a, int B, hipStream_t s);
hipError_t launch_decode(int G, int TC, bool tasq, const DecodeArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_rope_table(double theta, int D, int n_pos, void* table, hipStream_t s);
// Mean, then covariance, of the block-stacked scaled keys (needs sigma
// written first); T_c*D a multiple of 64 and at most 1024.
hipError_t launch_tasq_stats(const TasqStatsArgs& a, hipStream_t s);
// Weighted k-means update: accumulate (G in {16, 32}, K <= 256), then
// e = bf16(sums / wsum) for the n = H*n_blk*K*G codebook entries with wsum > 0.
hipError_t launch_kmeans_accumulate(const KmeansArgs& a, int B, bool tasq, hipStream_t s);
hipError_t launch_kmeans_finalize(const double* sums, const double* wsum, uint16_t* cb, int64_t n, int G,
                                  hipStream_t s);
hipError_t launch_decode_fast(int G, const DecodeArgs& a, hipStream_t s);
// T_c = 4, no pre-transform; one workgroup per (split, q-head, batch x served
// step).
hipError_t launch_decode_step(int G, const DecodeArgs& a, hipStream_t s);
// T_c = 4, no pre-transform, hpw in {2, 4} q-heads of a GQA group per
// workgroup; grid (n_split, Hq/hpw, B x blocks)
hipError_t launch_decode_gqa(int G, int hpw, const DecodeArgs& a, hipStream_t s);
// T_c = 4 with the channel pre-transform (keys); one q-head per workgroup;
// grid (n_split, Hq, B x served blocks); sigma must be 4-byte aligned.  one:
// the variant for a single served step (n_steps = 1), which computes only
// that step.
hipError_t launch_decode_tasq(int G, bool one, const DecodeArgs& a, hipStream_t s);

constexpr int kDecodeThreads = 256;
// threads per workgroup of decode_tasq_kernel<C, NSL>: at c = 4 one workgroup
// per CU, whose codebook copies fill most of the LDS (12 waves with every step
// of the block served, 16 with one served step); at c = 8 workgroups of 4 waves
constexpr int tasq_threads(int C, int NSL) { return C == 4 ? (NSL == 2 ? 768 : 1024) : kDecodeThreads; }
constexpr int kEncodeThreads = 256;
constexpr int kEncodeTokens = 128;  // tokens per encode workgroup

// fused decode for G = 16, T_c = 4 (c = 4), D = 128, plain keys
hipError_t launch_decode_half(const DecodeArgs& a, hipStream_t s);
// T_c = 1, G = 16 (per-step codebooks of 16 channels), no pre-transform; grid
// (n_split, Hq, B x served steps)
hipError_t launch_decode_cq(const DecodeArgs& a, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, hipStream_t s);   // p[0..n) = 0
hipError_t launch_rope_table_f32(float* tab, int n_pos, int D, double theta, hipStream_t s);
// forward (out, lse) or backward (delta, zeroed then accumulated codebook
// gradients, dq); C = G / T_c in {2, 4, 8, 16, 32}; C = 0: the precise cache
// (xk, xv), whose backward adds the key and value gradients into dxk, dxv
hipError_t launch_prefill(const PrefillArgs& a, int C, bool backward, hipStream_t s);
// omega of every joint vector (sum of the squared gradients of its G
// coordinates), for keys (with the pre-transform's scale and permutation
// when a.perm is set) and values
struct FisherArgs {
  const float* dk;            // fp32 [B][H][T][N_x][D] gradients of the pre-RoPE keys
  const float* dv;            // and of the values
  const float* w;             // keys' pre-transform or null
  const int16_t* perm;
  const uint16_t* sigma;      // fp16 [B][sig_cap][T]
  int32_t sig_cap;
  float* wk;                  // fp32 [B][H][n_blk][N][D/c]
  float* wv;
  int32_t B, H, T, T_c, n_blk, G, N, N_x, D;
};
hipError_t launch_fisher(const FisherArgs& a, hipStream_t s);

}  // namespace loopvq
