// Host side of the LoopVQ C ABI: argument checks, launch geometry, errors.
// Every check runs before the first HIP call; no C++ exception leaves here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/loopvq.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

loopvq_status fail(loopvq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

loopvq_status hip_fail(hipError_t e, const char* what) {
  return fail(LOOPVQ_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

// Geometry shared by both calls.
loopvq_status check_geom(const loopvq_geom* g) {
  if (!g) return fail(LOOPVQ_EINVAL, "geometry pointer is NULL");
  if (g->D < 2 || g->D % 2) return fail(LOOPVQ_EINVAL, "D=%d must be even and >= 2", g->D);
  if (g->T < 1 || g->T_c < 1 || g->T % g->T_c)
    return fail(LOOPVQ_EINVAL, "T=%d must be a positive multiple of T_c=%d", g->T, g->T_c);
  if (g->G < 1 || g->G % g->T_c)
    return fail(LOOPVQ_EINVAL, "G=%d must be a positive multiple of T_c=%d", g->G, g->T_c);
  const int c = g->G / g->T_c;
  if (g->D % c) return fail(LOOPVQ_EINVAL, "D=%d must be a multiple of c=G/T_c=%d", g->D, c);
  if (g->K < 2 || g->K > 256) return fail(LOOPVQ_EINVAL, "K=%d must be in [2, 256]", g->K);
  if (g->n_kv_heads < 1 || g->n_q_heads < 1 || g->n_q_heads % g->n_kv_heads)
    return fail(LOOPVQ_EINVAL, "n_q_heads=%d must be a positive multiple of n_kv_heads=%d",
                g->n_q_heads, g->n_kv_heads);
  if (!(g->rope_theta > 0.f) || !std::isfinite(g->rope_theta))
    return fail(LOOPVQ_EINVAL, "rope_theta must be positive and finite");
  if (g->D != 128) return fail(LOOPVQ_ENOTSUP, "this build supports D=128 only (got %d)", g->D);
  if (g->G != 16 && g->G != 32) return fail(LOOPVQ_ENOTSUP, "this build supports G in {16, 32} (got %d)", g->G);
  if (!pow2(g->T_c) || g->T_c > 8) return fail(LOOPVQ_ENOTSUP, "this build supports T_c in {1,2,4,8} (got %d)", g->T_c);
  if ((g->D / 2) % c) return fail(LOOPVQ_ENOTSUP, "c=%d must divide D/2", c);
  return LOOPVQ_OK;
}

loopvq_status check_pt(const loopvq_pretransform* pt, int B, int tok_end, bool need_sigma_write) {
  if (!pt) return LOOPVQ_OK;
  if (!pt->w || !pt->perm || !pt->sigma) return fail(LOOPVQ_EINVAL, "pre-transform has a NULL pointer");
  if (pt->N_cap < tok_end)
    return fail(LOOPVQ_EINVAL, "pre-transform sigma capacity %d < %d tokens", pt->N_cap, tok_end);
  (void)B;
  (void)need_sigma_write;
  return LOOPVQ_OK;
}

enum class DecodeKernel { kGeneric, kFast, kStep, kGqa, kTasq, kCq };

struct DecodePlan {
  int n_blk_serv, blk0, n_split, tok_per_split;
  int hpw;              // q-heads per workgroup of the MFMA kernel (2 or 4; 1: other kernels)
  DecodeKernel kernel;
  size_t ws_bytes;
};

DecodePlan plan_decode(const loopvq_geom* g, int B, int N, int step0, int n_steps, bool tasq) {
  DecodePlan p;
  p.blk0 = step0 / g->T_c;
  const int blk1 = (step0 + n_steps - 1) / g->T_c;
  p.n_blk_serv = blk1 - p.blk0 + 1;
  const int gqa = g->n_q_heads / g->n_kv_heads;
  p.hpw = gqa % 4 == 0 ? 4 : (gqa % 2 == 0 ? 2 : 1);
  // Blocks of four steps: GQA groups of two or four q-heads use the MFMA
  // kernel (two or four heads x the served steps as score rows; a single
  // served step reads only its own codeword slices); other groups use the
  // single-step kernel for one served step (one workgroup per step) and
  // otherwise the multi-step kernel, which decodes each index row once for all
  // steps of its block.  Pre-transformed keys in blocks of four steps have
  // their own kernel (one q-head per workgroup; one served step takes its
  // one-step variant); other block lengths use the
  // generic kernel, except per-step codebooks (T_c = 1) of 16 channels, which
  // have their own kernel.
  if (g->T_c == 1 && g->G == 16 && !tasq)
    p.kernel = DecodeKernel::kCq;
  else if (g->T_c != 4)
    p.kernel = DecodeKernel::kGeneric;
  else if (tasq)
    p.kernel = DecodeKernel::kTasq;
  else if (p.hpw > 1)
    p.kernel = DecodeKernel::kGqa;
  else if (n_steps == 1)
    p.kernel = DecodeKernel::kStep;
  else
    p.kernel = DecodeKernel::kFast;
  long long wgs;
  int target;   // about one resident round of workgroups
  switch (p.kernel) {
    case DecodeKernel::kStep:
      wgs = (long long)B * g->n_q_heads * n_steps;
      target = 1024;                       // 95 VGPRs: 4 per CU
      break;
    case DecodeKernel::kGqa:
      wgs = (long long)B * (g->n_q_heads / p.hpw) * p.n_blk_serv;
      target = 512;
      break;
    case DecodeKernel::kTasq:
      wgs = (long long)B * g->n_q_heads * p.n_blk_serv;
      // c = 4: one workgroup per CU (its codebook copies fill most of the
      // LDS: 12 waves for several steps, 16 for one); c = 8: several steps two
      // workgroups of 4 waves per CU (three fit, and measured slower), one
      // served step four (at most 128 VGPRs, 35 KB LDS)
      target = g->G == 16 ? 256 : (n_steps == 1 ? 1024 : 512);
      break;
    default:
      wgs = (long long)B * g->n_q_heads * p.n_blk_serv;
      target = 512;                        // 255 VGPRs: 2 per CU
  }
  long long ns = (target + wgs - 1) / wgs;
  const long long max_by_tokens = N > 0 ? (N + 255) / 256 : 1;
  if (ns > max_by_tokens) ns = max_by_tokens;
  if (ns < 1) ns = 1;
  p.n_split = (int)ns;
  p.tok_per_split = N > 0 ? (N + p.n_split - 1) / p.n_split : 0;
  p.ws_bytes = (size_t)B * g->n_q_heads * n_steps * p.n_split * (g->D + 1) * sizeof(float);
  return p;
}

// Split partials of loopvq_decode_attn_noalloc: a static device array (one
// copy per GPU, kept until the process ends).  In host code `scratch` names a
// host-side stand-in; its device address is taken once per device with
// hipGetSymbolAddress and only that address is passed to kernels.
constexpr size_t kScratchBytes = LOOPVQ_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch address (looked up on the first call on a device,
// with that device current).
loopvq_status scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(LOOPVQ_ENOTSUP, "device %d is beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LOOPVQ_OK;
}

}  // namespace

extern "C" {

const char* loopvq_last_error(void) { return g_err; }

int32_t loopvq_abi_version(void) { return LOOPVQ_ABI_VERSION; }

loopvq_status loopvq_encode(const loopvq_geom* g, const void* x, const int64_t x_strides[4],
                            const void* codebook, int32_t B, int32_t N, int32_t tok0,
                            uint8_t* idx, int32_t N_cap, const loopvq_pretransform* pt,
                            void* stream) {
  g_err[0] = 0;
  loopvq_status st = check_geom(g);
  if (st != LOOPVQ_OK) return st;
  if (B < 0 || N < 0 || tok0 < 0) return fail(LOOPVQ_EINVAL, "B=%d, N=%d, tok0=%d must be >= 0", B, N, tok0);
  if ((long long)tok0 + N > N_cap) return fail(LOOPVQ_EINVAL, "tok0 + N = %lld exceeds N_cap=%d", (long long)tok0 + N, N_cap);
  if (N == 0 || B == 0) return LOOPVQ_OK;
  if (!x || !x_strides || !codebook || !idx) return fail(LOOPVQ_EINVAL, "NULL tensor pointer");
  for (int i = 0; i < 4; ++i)
    if (x_strides[i] <= 0 || x_strides[i] % 8)
      return fail(LOOPVQ_EINVAL, "x_strides[%d]=%lld must be a positive multiple of 8", i, (long long)x_strides[i]);
  if (x_strides[3] < g->D) return fail(LOOPVQ_EINVAL, "token stride %lld < D", (long long)x_strides[3]);
  if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(codebook) % 16)
    return fail(LOOPVQ_EINVAL, "x and codebook must be 16-byte aligned");
  st = check_pt(pt, B, tok0 + N, true);
  if (st != LOOPVQ_OK) return st;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  loopvq::EncodeArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.xs0 = x_strides[0];
  a.xs1 = x_strides[1];
  a.xs2 = x_strides[2];
  a.xs3 = x_strides[3];
  a.cb = static_cast<const uint16_t*>(codebook);
  a.idx = idx;
  a.H = g->n_kv_heads;
  a.n_blk = g->T / g->T_c;
  a.K = g->K;
  a.T = g->T;
  a.N = N;
  a.tok0 = tok0;
  a.N_cap = N_cap;
  if (pt) {
    loopvq::SigmaArgs sa{};
    sa.x = a.x;
    sa.xs0 = a.xs0;
    sa.xs1 = a.xs1;
    sa.xs2 = a.xs2;
    sa.xs3 = a.xs3;
    sa.H = a.H;
    sa.T = a.T;
    sa.N = N;
    sa.tok0 = tok0;
    sa.sig_cap = pt->N_cap;
    sa.sigma = pt->sigma;
    hipError_t e = loopvq::launch_sigma(sa, B, s);
    if (e != hipSuccess) return hip_fail(e, "sigma launch");
    a.w = pt->w;
    a.perm = pt->perm;
    a.sigma = pt->sigma;
    a.sig_cap = pt->N_cap;
  }
  hipError_t e = loopvq::launch_encode(g->G, g->T_c, pt != nullptr, a, B, s);
  if (e != hipSuccess) return hip_fail(e, "encode launch");
  return LOOPVQ_OK;
}

loopvq_status loopvq_rope_table(float theta, int32_t D, int32_t n_pos, void* table, void* stream) {
  g_err[0] = 0;
  if (!table) return fail(LOOPVQ_EINVAL, "table is NULL");
  if (n_pos < 1) return fail(LOOPVQ_EINVAL, "n_pos=%d must be >= 1", n_pos);
  if (D < 8 || D % 8) return fail(LOOPVQ_EINVAL, "D=%d must be a positive multiple of 8", D);
  if (!(theta > 0.f) || !std::isfinite(theta)) return fail(LOOPVQ_EINVAL, "theta must be positive");
  hipError_t e = loopvq::launch_rope_table((double)theta, D, n_pos, table, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  return LOOPVQ_OK;
}

loopvq_status loopvq_tasq_covariance(const loopvq_geom* g, const void* x, const int64_t x_strides[4],
                                     int32_t B, int32_t N, const float* w, uint16_t* sigma, int32_t sig_cap,
                                     double* mean, double* cov, void* stream) {
  g_err[0] = 0;
  loopvq_status st = check_geom(g);
  if (st != LOOPVQ_OK) return st;
  if (B < 1 || N < 1) return fail(LOOPVQ_EINVAL, "B=%d and N=%d must be >= 1", B, N);
  if (!x || !x_strides || !w || !sigma || !mean || !cov) return fail(LOOPVQ_EINVAL, "NULL pointer");
  if (sig_cap < N) return fail(LOOPVQ_EINVAL, "sigma capacity %d < N=%d", sig_cap, N);
  for (int i = 0; i < 4; ++i)
    if (x_strides[i] <= 0 || x_strides[i] % 8)
      return fail(LOOPVQ_EINVAL, "x_strides[%d]=%lld must be a positive multiple of 8", i, (long long)x_strides[i]);
  if (x_strides[3] < g->D) return fail(LOOPVQ_EINVAL, "token stride %lld < D", (long long)x_strides[3]);
  if (reinterpret_cast<uintptr_t>(x) % 16) return fail(LOOPVQ_EINVAL, "x must be 16-byte aligned");
  if (g->T_c * g->D > 1024) return fail(LOOPVQ_ENOTSUP, "T_c*D=%d exceeds 1024", g->T_c * g->D);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  loopvq::SigmaArgs sa{};
  sa.x = static_cast<const uint16_t*>(x);
  sa.xs0 = x_strides[0];
  sa.xs1 = x_strides[1];
  sa.xs2 = x_strides[2];
  sa.xs3 = x_strides[3];
  sa.H = g->n_kv_heads;
  sa.T = g->T;
  sa.N = N;
  sa.tok0 = 0;
  sa.sig_cap = sig_cap;
  sa.sigma = sigma;
  hipError_t e = loopvq::launch_sigma(sa, B, s);
  if (e != hipSuccess) return hip_fail(e, "sigma launch");
  loopvq::TasqStatsArgs a{};
  a.x = sa.x;
  a.xs0 = sa.xs0;
  a.xs1 = sa.xs1;
  a.xs2 = sa.xs2;
  a.xs3 = sa.xs3;
  a.w = w;
  a.sigma = sigma;
  a.sig_cap = sig_cap;
  a.mean = mean;
  a.cov = cov;
  a.B = B;
  a.H = g->n_kv_heads;
  a.T = g->T;
  a.T_c = g->T_c;
  a.n_blk = g->T / g->T_c;
  a.N = N;
  a.D = g->D;
  e = loopvq::launch_tasq_stats(a, s);
  if (e != hipSuccess) return hip_fail(e, "covariance launch");
  return LOOPVQ_OK;
}

loopvq_status loopvq_tasq_pair_permutation(const double* cov, int32_t T_c, int32_t D, int32_t c, int16_t* perm) {
  g_err[0] = 0;
  if (!cov || !perm) return fail(LOOPVQ_EINVAL, "NULL pointer");
  if (T_c < 1 || D < 2 || D % 2 || c < 2 || c % 2 || D % c)
    return fail(LOOPVQ_EINVAL, "need T_c >= 1, even D, even c dividing D (T_c=%d, D=%d, c=%d)", T_c, D, c);
  if (D > 32767) return fail(LOOPVQ_EINVAL, "D=%d does not fit int16 channel numbers", D);
  const int F = T_c * D, HD = D / 2, per = c / 2;
  // correlation magnitudes folded over (step, step) and the two channels of
  // each RoPE pair
  std::vector<double> sd(F);
  for (int f = 0; f < F; ++f) {
    const double v = cov[(size_t)f * F + f];
    sd[f] = v > 0.0 ? std::sqrt(v) : 0.0;
  }
  std::vector<double> A((size_t)HD * HD, 0.0);
  for (int u = 0; u < HD; ++u)
    for (int v = u + 1; v < HD; ++v) {   // one value per unordered pair keeps exact ties exact
      double acc = 0.0;
      for (int si = 0; si < T_c; ++si)
        for (int sj = 0; sj < T_c; ++sj)
          for (int ca = 0; ca < 2; ++ca)
            for (int cb = 0; cb < 2; ++cb) {
              const int fa = si * D + u + ca * HD, fb = sj * D + v + cb * HD;
              const double den = sd[fa] * sd[fb];
              if (den > 0.0) acc += std::fabs(cov[(size_t)fa * F + fb] / den);
            }
      A[(size_t)u * HD + v] = acc;
      A[(size_t)v * HD + u] = acc;
    }
  // greedy groups of `per` pairs: seed = free pair with the largest affinity
  // to the other free pairs, then the free pair closest to the group; ties
  // go to the lowest pair number
  std::vector<char> used(HD, 0);
  int out = 0;
  for (int left = HD; left > 0; left -= per) {
    int seed = -1;
    double best = -1.0;
    for (int u = 0; u < HD; ++u) {
      if (used[u]) continue;
      double tot = 0.0;
      for (int v = 0; v < HD; ++v)
        if (!used[v]) tot += A[(size_t)u * HD + v];
      if (tot > best) {
        best = tot;
        seed = u;
      }
    }
    std::vector<int> group{seed};
    used[seed] = 1;
    while ((int)group.size() < per) {
      int nxt = -1;
      double bg = -1.0;
      for (int v = 0; v < HD; ++v) {
        if (used[v]) continue;
        double gsum = 0.0;
        for (int u : group) gsum += A[(size_t)v * HD + u];
        if (gsum > bg) {
          bg = gsum;
          nxt = v;
        }
      }
      group.push_back(nxt);
      used[nxt] = 1;
    }
    for (int u : group) {
      perm[out++] = (int16_t)u;
      perm[out++] = (int16_t)(u + HD);
    }
  }
  return LOOPVQ_OK;
}

loopvq_status loopvq_kmeans_accumulate(const loopvq_geom* g, const void* x, const int64_t x_strides[4],
                                      int32_t B, int32_t N, const uint8_t* idx, int32_t N_cap,
                                      const float* weight, const loopvq_pretransform* pt, double* sums,
                                      double* wsum, void* stream) {
  g_err[0] = 0;
  loopvq_status st = check_geom(g);
  if (st != LOOPVQ_OK) return st;
  if (B < 0 || N < 0) return fail(LOOPVQ_EINVAL, "B=%d and N=%d must be >= 0", B, N);
  if (N > N_cap) return fail(LOOPVQ_EINVAL, "N=%d exceeds N_cap=%d", N, N_cap);
  if (N == 0 || B == 0) return LOOPVQ_OK;
  if (!x || !x_strides || !idx || !sums || !wsum) return fail(LOOPVQ_EINVAL, "NULL pointer");
  for (int i = 0; i < 4; ++i)
    if (x_strides[i] <= 0) return fail(LOOPVQ_EINVAL, "x_strides[%d]=%lld must be positive", i, (long long)x_strides[i]);
  if (x_strides[3] < g->D) return fail(LOOPVQ_EINVAL, "token stride %lld < D", (long long)x_strides[3]);
  st = check_pt(pt, B, N, false);
  if (st != LOOPVQ_OK) return st;
  loopvq::KmeansArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.xs0 = x_strides[0];
  a.xs1 = x_strides[1];
  a.xs2 = x_strides[2];
  a.xs3 = x_strides[3];
  a.idx = idx;
  a.weight = weight;
  if (pt) {
    a.w = pt->w;
    a.perm = pt->perm;
    a.sigma = pt->sigma;
    a.sig_cap = pt->N_cap;
  }
  a.sums = sums;
  a.wsum = wsum;
  a.H = g->n_kv_heads;
  a.T = g->T;
  a.T_c = g->T_c;
  a.n_blk = g->T / g->T_c;
  a.K = g->K;
  a.G = g->G;
  a.N = N;
  a.N_cap = N_cap;
  a.D = g->D;
  hipError_t e = loopvq::launch_kmeans_accumulate(a, B, pt != nullptr, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "k-means accumulate launch");
  return LOOPVQ_OK;
}

loopvq_status loopvq_kmeans_finalize(const loopvq_geom* g, const double* sums, const double* wsum,
                                    void* codebook, void* stream) {
  g_err[0] = 0;
  loopvq_status st = check_geom(g);
  if (st != LOOPVQ_OK) return st;
  if (!sums || !wsum || !codebook) return fail(LOOPVQ_EINVAL, "NULL pointer");
  const int64_t n = (int64_t)g->n_kv_heads * (g->T / g->T_c) * g->K * g->G;
  hipError_t e = loopvq::launch_kmeans_finalize(sums, wsum, static_cast<uint16_t*>(codebook), n, g->G,
                                                reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "k-means finalize launch");
  return LOOPVQ_OK;
}

static loopvq_status check_decode_shape(const loopvq_geom* g, int32_t B, int32_t N, int32_t step0,
                                        int32_t n_steps) {
  loopvq_status st = check_geom(g);
  if (st != LOOPVQ_OK) return st;
  if (B < 0 || N < 0) return fail(LOOPVQ_EINVAL, "B=%d and N=%d must be >= 0", B, N);
  if (n_steps < 1 || step0 < 0 || step0 + n_steps > g->T)
    return fail(LOOPVQ_EINVAL, "step range [%d, %d) must lie in [0, T=%d)", step0, step0 + n_steps, g->T);
  return LOOPVQ_OK;
}

loopvq_status loopvq_decode_attn_workspace(const loopvq_geom* g, int32_t B, int32_t N,
                                           int32_t step0, int32_t n_steps, size_t* bytes) {
  g_err[0] = 0;
  loopvq_status st = check_decode_shape(g, B, N, step0, n_steps);
  if (st != LOOPVQ_OK) return st;
  if (!bytes) return fail(LOOPVQ_EINVAL, "bytes is NULL");
  // the caller may or may not pass a pre-transform: cover both plans
  *bytes = B > 0 ? std::max(plan_decode(g, B, N, step0, n_steps, false).ws_bytes,
                            plan_decode(g, B, N, step0, n_steps, true).ws_bytes)
                 : 0;
  return LOOPVQ_OK;
}

// The decode call with the split partials in `workspace`, or (from_scratch)
// in this device's static scratch array.
static loopvq_status decode_attn_impl(const loopvq_geom* g, const void* q, int32_t step0,
                                      int32_t n_steps, const uint8_t* k_idx, const uint8_t* v_idx,
                                      int32_t N_cap, const void* k_cb, const void* v_cb,
                                      const void* sink_k, const void* sink_v, int32_t n_s,
                                      const void* recent_k, const void* recent_v, int32_t n_r,
                                      int32_t R_cap, int32_t B, int32_t N, const int32_t* seq_len,
                                      const loopvq_pretransform* pt, const void* rope_table,
                                      int32_t n_pos, float* out, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream, bool from_scratch) {
  g_err[0] = 0;
  loopvq_status st = check_decode_shape(g, B, N, step0, n_steps);
  if (st != LOOPVQ_OK) return st;
  if (n_s < 0) return fail(LOOPVQ_EINVAL, "n_s=%d must be >= 0", n_s);
  if (n_r < 0 || n_r > R_cap) return fail(LOOPVQ_EINVAL, "n_r=%d must lie in [0, R_cap=%d]", n_r, R_cap);
  if (N > N_cap) return fail(LOOPVQ_EINVAL, "N=%d exceeds N_cap=%d", N, N_cap);
  if (B == 0) return LOOPVQ_OK;
  if (!q || !k_cb || !v_cb || !rope_table || !out) return fail(LOOPVQ_EINVAL, "NULL tensor pointer");
  if (N > 0 && (!k_idx || !v_idx)) return fail(LOOPVQ_EINVAL, "NULL index pointer");
  if (n_s > 0 && (!sink_k || !sink_v)) return fail(LOOPVQ_EINVAL, "NULL sink pointer with n_s=%d", n_s);
  if (n_r > 0 && (!recent_k || !recent_v)) return fail(LOOPVQ_EINVAL, "NULL recent-window pointer with n_r=%d", n_r);
  if ((long long)n_s + N + n_r > n_pos)
    return fail(LOOPVQ_EINVAL, "rope table has %d positions, need n_s + N + n_r = %lld", n_pos,
                (long long)n_s + N + n_r);
  {
    const void* al[] = {q, k_idx, v_idx, k_cb, v_cb, sink_k, sink_v, recent_k, recent_v, rope_table,
                        from_scratch ? nullptr : workspace};
    for (const void* p : al)
      if (reinterpret_cast<uintptr_t>(p) % 16)
        return fail(LOOPVQ_EINVAL, "tensor pointers must be 16-byte aligned");
  }
  st = check_pt(pt, B, N, false);
  if (st != LOOPVQ_OK) return st;
  const DecodePlan p = plan_decode(g, B, N, step0, n_steps, pt != nullptr);
  if (p.kernel == DecodeKernel::kTasq && reinterpret_cast<uintptr_t>(pt->sigma) % 4)
    return fail(LOOPVQ_EINVAL, "pre-transform sigma must be 4-byte aligned");
  // byte offsets of the index rows, sigma and the table are 32-bit in the
  // pre-transform kernel
  if (p.kernel == DecodeKernel::kTasq &&
      ((long long)N_cap * (g->D / (g->G / g->T_c)) >= (1ll << 31) || (long long)pt->N_cap * g->T * 2 >= (1ll << 31) ||
       (long long)n_pos * g->D * 2 >= (1ll << 31)))
    return fail(LOOPVQ_ENOTSUP, "N_cap=%d or n_pos=%d too large for 32-bit offsets", N_cap, n_pos);
  if (from_scratch) {
    if (p.ws_bytes > kScratchBytes)
      return fail(LOOPVQ_EWORKSPACE, "this shape needs %zu bytes of split partials; the allocation-free call "
                  "holds at most %zu (use loopvq_decode_attn with a workspace)", p.ws_bytes, kScratchBytes);
    st = scratch_for_current_device(&workspace);
    if (st != LOOPVQ_OK) return st;
    workspace_bytes = kScratchBytes;
  } else if (!workspace || workspace_bytes < p.ws_bytes) {
    return fail(LOOPVQ_EWORKSPACE, "workspace of %zu bytes needed (got %zu)", p.ws_bytes, workspace_bytes);
  }

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  loopvq::DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kidx = k_idx;
  a.vidx = v_idx;
  a.kcb = static_cast<const uint16_t*>(k_cb);
  a.vcb = static_cast<const uint16_t*>(v_cb);
  a.sk = static_cast<const uint16_t*>(sink_k);
  a.sv = static_cast<const uint16_t*>(sink_v);
  a.rk = static_cast<const uint16_t*>(recent_k);
  a.rv = static_cast<const uint16_t*>(recent_v);
  a.n_r = n_r;
  a.r_cap = R_cap;
  a.seq_len = seq_len;
  if (pt) {
    a.w = pt->w;
    a.perm = pt->perm;
    a.sigma = pt->sigma;
    a.sig_cap = pt->N_cap;
  }
  a.rope = rope_table;
  a.ws = static_cast<float*>(workspace);
  a.B = B;
  a.H = g->n_kv_heads;
  a.Hq = g->n_q_heads;
  a.T = g->T;
  a.n_blk = g->T / g->T_c;
  a.K = g->K;
  a.N = N;
  a.N_cap = N_cap;
  a.n_s = n_s;
  a.step0 = step0;
  a.n_steps = n_steps;
  a.n_split = p.n_split;
  a.gqa = g->n_q_heads / g->n_kv_heads;
  a.blk0 = p.blk0;
  a.n_blk_serv = p.n_blk_serv;
  a.tok_per_split = p.tok_per_split;
  a.qscale = (float)(1.4426950408889634 / std::sqrt((double)g->D));
  a.theta = g->rope_theta;
  a.n_pos = n_pos;
  // One context split: the pre-transform, GQA and c = 4 multi-step kernels
  // write out / lse themselves and no merge kernel runs.
  const bool direct = p.n_split == 1 && (p.kernel == DecodeKernel::kTasq || p.kernel == DecodeKernel::kGqa ||
                                         (p.kernel == DecodeKernel::kFast && g->G == 16));
  if (direct) {
    a.out = out;
    a.lse = lse;
  }
  // Blocks of four steps (0.5 and 0.25 bit, with or without the key
  // pre-transform): the specialised kernels chosen by the plan; every other
  // geometry: the generic one.
  hipError_t e;
  if (p.kernel == DecodeKernel::kGeneric)
    e = loopvq::launch_decode(g->G, g->T_c, pt != nullptr, a, s);
  else if (p.kernel == DecodeKernel::kCq)
    e = loopvq::launch_decode_cq(a, s);
  else if (p.kernel == DecodeKernel::kTasq)
    e = loopvq::launch_decode_tasq(g->G, n_steps == 1, a, s);
  else if (p.kernel == DecodeKernel::kGqa)
    e = loopvq::launch_decode_gqa(g->G, p.hpw, a, s);
  else if (p.kernel == DecodeKernel::kStep)
    e = loopvq::launch_decode_step(g->G, a, s);
  else
    e = loopvq::launch_decode_fast(g->G, a, s);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (direct) return LOOPVQ_OK;   // the kernel wrote out / lse
  loopvq::MergeArgs ma{};
  ma.ws = a.ws;
  ma.out = out;
  ma.lse = lse;
  ma.rows = B * g->n_q_heads * n_steps;
  ma.n_split = p.n_split;
  e = loopvq::launch_merge(ma, s);
  if (e != hipSuccess) return hip_fail(e, "merge launch");
  return LOOPVQ_OK;
}

loopvq_status loopvq_decode_attn(const loopvq_geom* g, const void* q, int32_t step0,
                                 int32_t n_steps, const uint8_t* k_idx, const uint8_t* v_idx,
                                 int32_t N_cap, const void* k_cb, const void* v_cb,
                                 const void* sink_k, const void* sink_v, int32_t n_s,
                                 const void* recent_k, const void* recent_v, int32_t n_r,
                                 int32_t R_cap, int32_t B, int32_t N, const int32_t* seq_len,
                                 const loopvq_pretransform* pt, const void* rope_table,
                                 int32_t n_pos, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return decode_attn_impl(g, q, step0, n_steps, k_idx, v_idx, N_cap, k_cb, v_cb, sink_k, sink_v, n_s, recent_k,
                          recent_v, n_r, R_cap, B, N, seq_len, pt, rope_table, n_pos, out, lse, workspace,
                          workspace_bytes, stream, false);
}

loopvq_status loopvq_decode_attn_noalloc(const loopvq_geom* g, const void* q, int32_t step0,
                                         int32_t n_steps, const uint8_t* k_idx, const uint8_t* v_idx,
                                         int32_t N_cap, const void* k_cb, const void* v_cb,
                                         const void* sink_k, const void* sink_v, int32_t n_s,
                                         const void* recent_k, const void* recent_v, int32_t n_r,
                                         int32_t R_cap, int32_t B, int32_t N, const int32_t* seq_len,
                                         const loopvq_pretransform* pt, const void* rope_table,
                                         int32_t n_pos, float* out, float* lse, void* stream) {
  return decode_attn_impl(g, q, step0, n_steps, k_idx, v_idx, N_cap, k_cb, v_cb, sink_k, sink_v, n_s, recent_k,
                          recent_v, n_r, R_cap, B, N, seq_len, pt, rope_table, n_pos, out, lse, nullptr, 0, stream,
                          true);
}

loopvq_status loopvq_rope_table_f32(float theta, int32_t D, int32_t n_pos, float* table, void* stream) {
  g_err[0] = 0;
  if (!table) return fail(LOOPVQ_EINVAL, "table is NULL");
  if (n_pos < 1) return fail(LOOPVQ_EINVAL, "n_pos=%d must be >= 1", n_pos);
  if (D < 2 || D % 2) return fail(LOOPVQ_EINVAL, "D=%d must be even and >= 2", D);
  if (!(theta > 0.f) || !std::isfinite(theta)) return fail(LOOPVQ_EINVAL, "theta must be positive");
  hipError_t e = loopvq::launch_rope_table_f32(table, n_pos, D, (double)theta, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  return LOOPVQ_OK;
}

static loopvq_status prefill_args(const loopvq_geom* g, const float* q, int32_t step0, int32_t n_steps,
                                  int32_t B, int32_t N, const uint8_t* k_idx, const uint8_t* v_idx,
                                  int32_t N_cap, const void* k_cb, const void* v_cb, const void* sink_k,
                                  const void* sink_v, int32_t n_s, const loopvq_pretransform* pt,
                                  const float* rope_table, int32_t n_pos, loopvq::PrefillArgs& a) {
  loopvq_status st = check_decode_shape(g, B, N, step0, n_steps);
  if (st != LOOPVQ_OK) return st;
  if (n_s < 0) return fail(LOOPVQ_EINVAL, "n_s=%d must be >= 0", n_s);
  if (N > N_cap) return fail(LOOPVQ_EINVAL, "N=%d exceeds N_cap=%d", N, N_cap);
  if (B > 0 && N > 0) {   // an empty call may pass NULL tensors
    if (!q || !k_idx || !v_idx || !k_cb || !v_cb || !rope_table)
      return fail(LOOPVQ_EINVAL, "NULL tensor pointer");
    if (n_s > 0 && (!sink_k || !sink_v)) return fail(LOOPVQ_EINVAL, "sinks are NULL with n_s=%d", n_s);
    if ((long long)n_s + N > n_pos) return fail(LOOPVQ_EINVAL, "rope table has %d positions, need %lld", n_pos,
                                                 (long long)n_s + N);
  }
  for (const void* p : {(const void*)q, (const void*)rope_table, sink_k, sink_v})
    if (reinterpret_cast<uintptr_t>(p) % 16) return fail(LOOPVQ_EINVAL, "q, rope_table and sinks must be 16-byte aligned");
  if (pt) {
    st = check_pt(pt, B, N, false);
    if (st != LOOPVQ_OK) return st;
  }
  a = loopvq::PrefillArgs{};
  if (pt) {
    a.w = pt->w;
    a.perm = pt->perm;
    a.sigma = static_cast<const uint16_t*>(pt->sigma);
    a.sig_cap = pt->N_cap;
  }
  a.q = q;
  a.kidx = k_idx;
  a.vidx = v_idx;
  a.kcb = static_cast<const uint16_t*>(k_cb);
  a.vcb = static_cast<const uint16_t*>(v_cb);
  a.sk = static_cast<const uint16_t*>(sink_k);
  a.sv = static_cast<const uint16_t*>(sink_v);
  a.rope = rope_table;
  a.B = B;
  a.H = g->n_kv_heads;
  a.Hq = g->n_q_heads;
  a.T = g->T;
  a.T_c = g->T_c;
  a.n_blk = g->T / g->T_c;
  a.K = g->K;
  a.G = g->G;
  a.N = N;
  a.N_cap = N_cap;
  a.n_s = n_s;
  a.step0 = step0;
  a.n_steps = n_steps;
  a.gqa = g->n_q_heads / g->n_kv_heads;
  a.scale = (float)(1.0 / std::sqrt((double)g->D));
  return LOOPVQ_OK;
}

loopvq_status loopvq_prefill_attn(const loopvq_geom* g, const float* q, int32_t step0, int32_t n_steps,
                                  int32_t B, int32_t N, const uint8_t* k_idx, const uint8_t* v_idx,
                                  int32_t N_cap, const void* k_cb, const void* v_cb, const void* sink_k,
                                  const void* sink_v, int32_t n_s, const loopvq_pretransform* pt,
                                  const float* rope_table, int32_t n_pos, float* out, float* lse, void* stream) {
  g_err[0] = 0;
  loopvq::PrefillArgs a;
  loopvq_status st = prefill_args(g, q, step0, n_steps, B, N, k_idx, v_idx, N_cap, k_cb, v_cb, sink_k, sink_v,
                                  n_s, pt, rope_table, n_pos, a);
  if (st != LOOPVQ_OK) return st;
  if (B == 0 || N == 0) return LOOPVQ_OK;
  if (!out || !lse) return fail(LOOPVQ_EINVAL, "out and lse must not be NULL");
  if (reinterpret_cast<uintptr_t>(out) % 16) return fail(LOOPVQ_EINVAL, "out must be 16-byte aligned");
  a.out = out;
  a.lse = lse;
  hipError_t e = loopvq::launch_prefill(a, g->G / g->T_c, false, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  return LOOPVQ_OK;
}

loopvq_status loopvq_prefill_attn_backward_workspace(const loopvq_geom* g, int32_t B, int32_t N,
                                                     int32_t step0, int32_t n_steps, size_t* bytes) {
  g_err[0] = 0;
  loopvq_status st = check_decode_shape(g, B, N, step0, n_steps);
  if (st != LOOPVQ_OK) return st;
  if (!bytes) return fail(LOOPVQ_EINVAL, "bytes is NULL");
  *bytes = (size_t)B * g->n_q_heads * n_steps * N * sizeof(float);
  return LOOPVQ_OK;
}

loopvq_status loopvq_prefill_attn_backward(const loopvq_geom* g, const float* q, int32_t step0,
                                           int32_t n_steps, int32_t B, int32_t N, const uint8_t* k_idx,
                                           const uint8_t* v_idx, int32_t N_cap, const void* k_cb,
                                           const void* v_cb, const void* sink_k, const void* sink_v,
                                           int32_t n_s, const loopvq_pretransform* pt, const float* rope_table,
                                           int32_t n_pos, const float* out, const float* lse, const float* d_out,
                                           float* d_q, float* d_k_cb, float* d_v_cb, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  loopvq::PrefillArgs a;
  loopvq_status st = prefill_args(g, q, step0, n_steps, B, N, k_idx, v_idx, N_cap, k_cb, v_cb, sink_k, sink_v,
                                  n_s, pt, rope_table, n_pos, a);
  if (st != LOOPVQ_OK) return st;
  if (!d_k_cb || !d_v_cb) return fail(LOOPVQ_EINVAL, "NULL codebook gradient");
  if (B > 0 && N > 0 && (!out || !lse || !d_out || !d_q)) return fail(LOOPVQ_EINVAL, "NULL tensor pointer");
  for (const void* p : {(const void*)out, (const void*)d_out, (const void*)d_q})
    if (reinterpret_cast<uintptr_t>(p) % 16) return fail(LOOPVQ_EINVAL, "out, d_out and d_q must be 16-byte aligned");
  const size_t need = (size_t)B * g->n_q_heads * n_steps * N * sizeof(float);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(LOOPVQ_EWORKSPACE, "workspace of %zu bytes < %zu", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return fail(LOOPVQ_EINVAL, "workspace must be 16-byte aligned");
  a.out = const_cast<float*>(out);
  a.lse = const_cast<float*>(lse);
  a.dout = d_out;
  a.dq = d_q;
  a.dkcb = d_k_cb;
  a.dvcb = d_v_cb;
  a.delta = static_cast<float*>(workspace);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (B == 0 || N == 0) {
    // nothing attends: the codebook gradients are zero
    const int64_t ncb = (int64_t)g->n_kv_heads * (g->T / g->T_c) * g->K * g->G;
    e = loopvq::launch_fill_f32(d_k_cb, ncb, s);
    if (e == hipSuccess) e = loopvq::launch_fill_f32(d_v_cb, ncb, s);
  } else {
    e = loopvq::launch_prefill(a, g->G / g->T_c, true, s);
  }
  if (e != hipSuccess) return hip_fail(e, "prefill attention backward launch");
  return LOOPVQ_OK;
}

static loopvq_status precise_args(const loopvq_geom* g, const float* q, int32_t step0, int32_t n_steps,
                                  int32_t B, int32_t N, const void* k, const void* v, int32_t N_x,
                                  const void* sink_k, const void* sink_v, int32_t n_s, const float* rope_table,
                                  int32_t n_pos, loopvq::PrefillArgs& a) {
  loopvq_status st = check_decode_shape(g, B, N, step0, n_steps);
  if (st != LOOPVQ_OK) return st;
  if (n_s < 0) return fail(LOOPVQ_EINVAL, "n_s=%d must be >= 0", n_s);
  if (N > N_x) return fail(LOOPVQ_EINVAL, "N=%d exceeds the cache's N_x=%d tokens", N, N_x);
  if (B > 0 && N > 0) {
    if (!q || !k || !v || !rope_table) return fail(LOOPVQ_EINVAL, "NULL tensor pointer");
    if (n_s > 0 && (!sink_k || !sink_v)) return fail(LOOPVQ_EINVAL, "sinks are NULL with n_s=%d", n_s);
    if ((long long)n_s + N > n_pos) return fail(LOOPVQ_EINVAL, "rope table has %d positions, need %lld", n_pos,
                                                 (long long)n_s + N);
  }
  for (const void* p : {(const void*)q, (const void*)rope_table, sink_k, sink_v, k, v})
    if (reinterpret_cast<uintptr_t>(p) % 16)
      return fail(LOOPVQ_EINVAL, "q, k, v, rope_table and sinks must be 16-byte aligned");
  a = loopvq::PrefillArgs{};
  a.q = q;
  a.xk = static_cast<const uint16_t*>(k);
  a.xv = static_cast<const uint16_t*>(v);
  a.N_x = N_x;
  a.sk = static_cast<const uint16_t*>(sink_k);
  a.sv = static_cast<const uint16_t*>(sink_v);
  a.rope = rope_table;
  a.B = B;
  a.H = g->n_kv_heads;
  a.Hq = g->n_q_heads;
  a.T = g->T;
  a.T_c = g->T_c;
  a.n_blk = g->T / g->T_c;
  a.K = g->K;
  a.G = g->G;
  a.N = N;
  a.N_cap = N_x;
  a.n_s = n_s;
  a.step0 = step0;
  a.n_steps = n_steps;
  a.gqa = g->n_q_heads / g->n_kv_heads;
  a.scale = (float)(1.0 / std::sqrt((double)g->D));
  return LOOPVQ_OK;
}

loopvq_status loopvq_precise_attn(const loopvq_geom* g, const float* q, int32_t step0, int32_t n_steps,
                                  int32_t B, int32_t N, const void* k, const void* v, int32_t N_x,
                                  const void* sink_k, const void* sink_v, int32_t n_s, const float* rope_table,
                                  int32_t n_pos, float* out, float* lse, void* stream) {
  g_err[0] = 0;
  loopvq::PrefillArgs a;
  loopvq_status st = precise_args(g, q, step0, n_steps, B, N, k, v, N_x, sink_k, sink_v, n_s, rope_table, n_pos, a);
  if (st != LOOPVQ_OK) return st;
  if (B == 0 || N == 0) return LOOPVQ_OK;
  if (!out || !lse) return fail(LOOPVQ_EINVAL, "out and lse must not be NULL");
  if (reinterpret_cast<uintptr_t>(out) % 16) return fail(LOOPVQ_EINVAL, "out must be 16-byte aligned");
  a.out = out;
  a.lse = lse;
  hipError_t e = loopvq::launch_prefill(a, 0, false, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "precise attention launch");
  return LOOPVQ_OK;
}

loopvq_status loopvq_precise_attn_backward(const loopvq_geom* g, const float* q, int32_t step0, int32_t n_steps,
                                           int32_t B, int32_t N, const void* k, const void* v, int32_t N_x,
                                           const void* sink_k, const void* sink_v, int32_t n_s,
                                           const float* rope_table, int32_t n_pos, const float* out,
                                           const float* lse, const float* d_out, float* d_q, float* d_k,
                                           float* d_v, void* workspace, size_t workspace_bytes, void* stream) {
  g_err[0] = 0;
  loopvq::PrefillArgs a;
  loopvq_status st = precise_args(g, q, step0, n_steps, B, N, k, v, N_x, sink_k, sink_v, n_s, rope_table, n_pos, a);
  if (st != LOOPVQ_OK) return st;
  if (B == 0 || N == 0) return LOOPVQ_OK;
  if (!out || !lse || !d_out || !d_q || !d_k || !d_v) return fail(LOOPVQ_EINVAL, "NULL tensor pointer");
  for (const void* p : {(const void*)out, (const void*)d_out, (const void*)d_q})
    if (reinterpret_cast<uintptr_t>(p) % 16) return fail(LOOPVQ_EINVAL, "out, d_out and d_q must be 16-byte aligned");
  const size_t need = (size_t)B * g->n_q_heads * n_steps * N * sizeof(float);
  if (!workspace || workspace_bytes < need)
    return fail(LOOPVQ_EWORKSPACE, "workspace of %zu bytes < %zu", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) % 16) return fail(LOOPVQ_EINVAL, "workspace must be 16-byte aligned");
  a.out = const_cast<float*>(out);
  a.lse = const_cast<float*>(lse);
  a.dout = d_out;
  a.dq = d_q;
  a.dxk = d_k;
  a.dxv = d_v;
  a.delta = static_cast<float*>(workspace);
  hipError_t e = loopvq::launch_prefill(a, 0, true, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "precise attention backward launch");
  return LOOPVQ_OK;
}

loopvq_status loopvq_fisher_weights(const loopvq_geom* g, const float* d_k, const float* d_v, int32_t B, int32_t N,
                                    int32_t N_x, const loopvq_pretransform* pt, float* omega_k, float* omega_v,
                                    void* stream) {
  g_err[0] = 0;
  loopvq_status st = check_geom(g);
  if (st != LOOPVQ_OK) return st;
  if (B < 0 || N < 0) return fail(LOOPVQ_EINVAL, "B=%d and N=%d must be >= 0", B, N);
  if (N > N_x) return fail(LOOPVQ_EINVAL, "N=%d exceeds N_x=%d", N, N_x);
  if (B == 0 || N == 0) return LOOPVQ_OK;
  if (!d_k || !d_v || !omega_k || !omega_v) return fail(LOOPVQ_EINVAL, "NULL tensor pointer");
  st = check_pt(pt, B, N, false);
  if (st != LOOPVQ_OK) return st;
  loopvq::FisherArgs a{};
  a.dk = d_k;
  a.dv = d_v;
  if (pt) {
    a.w = pt->w;
    a.perm = pt->perm;
    a.sigma = pt->sigma;
    a.sig_cap = pt->N_cap;
  }
  a.wk = omega_k;
  a.wv = omega_v;
  a.B = B;
  a.H = g->n_kv_heads;
  a.T = g->T;
  a.T_c = g->T_c;
  a.n_blk = g->T / g->T_c;
  a.G = g->G;
  a.N = N;
  a.N_x = N_x;
  a.D = g->D;
  hipError_t e = loopvq::launch_fisher(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "importance weight launch");
  return LOOPVQ_OK;
}

}  // extern "C"
