// Measurement helpers (not part of the LoopVQ ABI), built into
// libloopvq_calib.so:
//   * a plain device-to-device copy and a plain streaming read, both with
//     16-byte accesses per lane.  The benchmark times them to give the HBM
//     stream rates of this device, and the hardware byte counters
//     (FETCH_SIZE, WRITE_SIZE) read on them give the scale that turns the
//     counters of the LoopVQ kernels into bytes;
//   * on-chip ceilings of the resources the decode and encode kernels use:
//     LDS reads in the access patterns of the codebook gathers, packed-fp16
//     and fp32 vector arithmetic, and bf16 matrix-core products.  Each kernel
//     repeats independent operations from many waves per CU and folds the
//     results into one word per thread so nothing is optimised away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace loopvq_calib {

__global__ __launch_bounds__(256) void calib_copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         uint64_t n16) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(256) void calib_read_kernel(const uint4* __restrict__ src, uint64_t n16,
                                                         uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per thread keeps the loads live; the sink holds gridDim.x * 256 words
  sink[(uint64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// ---- LDS read ceilings.  A 32 KB table per workgroup (four workgroups, 16
// waves, per CU); 16 independent reads per lane per iteration.  Byte
// offsets are fixed per lane (16 per lane, from a hash) and xor-ed per
// iteration with a uniform multiple of 256 below 32 KB, which keeps every
// offset inside the table and its LDS bank unchanged.
//   mode 0: ds_read_b128, lane l reads slot l of a 1 KB row (no conflicts);
//   mode 1: ds_read_b128 at random 16-byte slots of the table;
//   mode 2: ds_read_b128 of codeword halves: random row of 48 bytes, half
//           chosen by the wave (the c = 4 decode's layout);
//   mode 3: ds_read_b64 at random 8-byte slots;
//   mode 4: ds_read_b64_tr_b16 at random 8-byte slots (transposed reads of
//           the matrix-core decode);
//   mode 5: ds_read_b128 of codeword halves, lanes 2i and 2i+1 reading the
//           two halves of one random 32-byte codeword (the pre-transform
//           decode's layout);
//   mode 6: as mode 5 with a 48-byte codeword stride;
//   mode 7: ds_bpermute_b32 from random source lanes (crossbar reads).
constexpr int kLdsBytes = 32768;

template <int MODE>
__global__ __launch_bounds__(256) void calib_lds_kernel(uint32_t* __restrict__ sink, int iters) {
  __shared__ __attribute__((aligned(16))) uint4 s[kLdsBytes / 16];
  for (int i = threadIdx.x; i < kLdsBytes / 16; i += 256) s[i] = make_uint4(i, i * 3u, i * 7u, i * 11u);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = 0x9e3779b9u * (threadIdx.x + 1) + blockIdx.x * 7919u;
  uint32_t off[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    if (MODE == 0) off[j] = (uint32_t)(lane * 16 + j * 1024) & (kLdsBytes - 1);
    else if (MODE == 1) off[j] = (x & (kLdsBytes / 16 - 1)) * 16;
    else if (MODE == 2) off[j] = (x & 255u) * 48 + 16 * (wave & 1);
    else if (MODE == 5 || MODE == 6) {
      // the two lanes of a pair draw the same codeword
      const uint32_t row = __shfl_xor((int)(x & 255u), 1) & 255u;
      const uint32_t mine = (lane & 1) ? row : (x & 255u);
      off[j] = mine * (MODE == 5 ? 32 : 48) + 16 * (lane & 1);
    } else if (MODE == 7) off[j] = (x & 63u) * 4;
    else off[j] = (x & (kLdsBytes / 8 - 1)) * 8;
  }
  const char* base = reinterpret_cast<const char*>(s);
  uint32_t a0 = 0, a1 = 0;
  for (int it = 0; it < iters; ++it) {
    // modes 5 and 6 add a multiple of 768 (pairs stay on one codeword, banks
    // unchanged, offsets below 24 KB); the others xor a multiple of 256
    const uint32_t u = (MODE == 5 || MODE == 6) ? ((uint32_t)(it * 37) & 15u) * 768u
                                                 : ((uint32_t)(it * 37) & 127u) * 256u;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t o = (MODE == 5 || MODE == 6) ? off[j] + u : off[j] ^ u;
      if constexpr (MODE <= 2 || MODE == 5 || MODE == 6) {
        const uint4 v = *reinterpret_cast<const uint4*>(base + o);
        (j & 1 ? a1 : a0) += v.x + v.y + v.z + v.w;
      } else if constexpr (MODE == 3) {
        const uint2 v = *reinterpret_cast<const uint2*>(base + o);
        (j & 1 ? a1 : a0) += v.x + v.y;
      } else if constexpr (MODE == 7) {
        // source lane varies per iteration through the uniform xor (low 8 bits unchanged: o & 255)
        (j & 1 ? a1 : a0) += (uint32_t)__builtin_amdgcn_ds_bpermute((int)(o & 255u), (int)o);
      } else {
        typedef short s4_t __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s4_t lds_s4;
        const s4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4*)((__attribute__((address_space(3))) char*)(__attribute__((address_space(3))) void*)s + o));
        const uint2 w = __builtin_bit_cast(uint2, v);
        (j & 1 ? a1 : a0) += w.x + w.y;
      }
    }
  }
  sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = a0 ^ a1;
}

// ---- vector-unit ceilings: 16 independent chains per lane.
//   mode 0: v_pk_fma_f16 (two fp16 FMAs per lane per instruction);
//   mode 1: v_dot2_f32_f16 (two fp16 products summed into fp32);
//   mode 2: v_fma_f32.
//   modes 3-8 (instruction issue rates of the selection and softmax steps;
//   each instruction written out so the compiler cannot substitute another):
//   v_min3_f32, v_med3_f32, v_perm_b32, v_mov_b32 with a DPP row shuffle,
//   v_exp_f32, v_add_f32.
template <int MODE>
__global__ __launch_bounds__(256) void calib_valu_kernel(uint32_t* __restrict__ sink, int iters) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const float f = 1.0f + (float)(threadIdx.x & 7) * 0.001f;
  uint32_t res = 0;
  if constexpr (MODE == 0) {
    h2_t acc[16];
    const h2_t m = {(_Float16)0.5f, (_Float16)0.5f}, c = {(_Float16)0.25f, (_Float16)(0.25f * f)};
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = h2_t{(_Float16)(f * j), (_Float16)f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = acc[j] * m + c;
#pragma unroll
    for (int j = 0; j < 16; ++j) res ^= __builtin_bit_cast(uint32_t, acc[j]);
  } else if constexpr (MODE == 1) {
    float acc[16];
    const h2_t a = {(_Float16)0.5f, (_Float16)(0.25f * f)}, b = {(_Float16)0.125f, (_Float16)0.5f};
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = f * j;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_fdot2(a, b, acc[j], false);
#pragma unroll
    for (int j = 0; j < 16; ++j) res ^= __float_as_uint(acc[j]);
  } else if constexpr (MODE == 2) {
    float acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = f * j;
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[j] = fmaf(acc[j], 0.5f, f);
#pragma unroll
    for (int j = 0; j < 16; ++j) res ^= __float_as_uint(acc[j]);
  } else {
    uint32_t acc[16];
    const uint32_t b = __float_as_uint(f), c = __float_as_uint(0.5f * f);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = __float_as_uint(f * (float)(j + 1));
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if constexpr (MODE == 3)
          asm volatile("v_min3_f32 %0, %0, %1, %2" : "+v"(acc[j]) : "v"(b), "v"(c));
        else if constexpr (MODE == 4)
          asm volatile("v_med3_f32 %0, %0, %1, %2" : "+v"(acc[j]) : "v"(b), "v"(c));
        else if constexpr (MODE == 5)
          asm volatile("v_perm_b32 %0, %0, %1, %2" : "+v"(acc[j]) : "v"(b), "v"(c));
        else if constexpr (MODE == 6)
          asm volatile("v_mov_b32_dpp %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf" : "+v"(acc[j]));
        else if constexpr (MODE == 7)
          asm volatile("v_exp_f32 %0, %0" : "+v"(acc[j]));
        else
          asm volatile("v_add_f32 %0, %0, %1" : "+v"(acc[j]) : "v"(b));
      }
#pragma unroll
    for (int j = 0; j < 16; ++j) res ^= acc[j];
  }
  sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = res;
}

// ---- matrix-core ceilings: four independent accumulator chains per wave.
//   mode 0: v_mfma_f32_16x16x32_bf16 (16384 flop per instruction);
//   mode 1: v_mfma_f32_32x32x16_bf16 (32768 flop per instruction).
template <int MODE>
__global__ __launch_bounds__(256) void calib_mfma_kernel(uint32_t* __restrict__ sink, int iters) {
  typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
  bf8_t a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(0.001f * (float)((threadIdx.x + j) & 15));
    b[j] = (__bf16)(0.002f * (float)((threadIdx.x * 3 + j) & 15));
  }
  uint32_t res = 0;
  if constexpr (MODE == 0) {
    typedef float f4_t __attribute__((ext_vector_type(4)));
    f4_t acc[4] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) res ^= __float_as_uint(acc[j][e]);
  } else if constexpr (MODE == 1) {
    typedef float f16_t __attribute__((ext_vector_type(16)));
    f16_t acc[4] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) res ^= __float_as_uint(acc[j][e]);
  } else {
    // the 32x32x8 bf16 product (four bf16 per lane) the encode uses for its
    // norm terms
    typedef float f16_t __attribute__((ext_vector_type(16)));
    typedef short s4_t __attribute__((ext_vector_type(4)));
    const s4_t a4 = {__builtin_bit_cast(short, a[0]), __builtin_bit_cast(short, a[1]), __builtin_bit_cast(short, a[2]),
                     __builtin_bit_cast(short, a[3])};
    const s4_t b4 = {__builtin_bit_cast(short, b[0]), __builtin_bit_cast(short, b[1]), __builtin_bit_cast(short, b[2]),
                     __builtin_bit_cast(short, b[3])};
    f16_t acc[4] = {};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(a4, b4, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) res ^= __float_as_uint(acc[j][e]);
  }
  sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = res;
}

int grid_for(uint64_t n16) {
  const uint64_t want = (n16 + 255) / 256;
  return (int)(want < 8192 ? (want ? want : 1) : 8192);
}

}  // namespace loopvq_calib

using namespace loopvq_calib;

extern "C" {

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) from src to
// dst on `stream`.  Returns 0, or -1 for bad arguments, -3 for a launch error.
int loopvq_calib_copy(const void* src, void* dst, uint64_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
    return -1;
  const uint64_t n16 = bytes / 16;
  hipLaunchKernelGGL(calib_copy_kernel, dim3(grid_for(n16)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n16);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// Number of uint32 words the sink of loopvq_calib_read must hold for `bytes`.
uint64_t loopvq_calib_read_sink_words(uint64_t bytes) { return (uint64_t)grid_for(bytes / 16) * 256; }

// Reads `bytes` (a multiple of 16, src 16-byte aligned) and writes one word
// per thread to sink.  Returns 0, -1 for bad arguments, -3 for a launch error.
int loopvq_calib_read(const void* src, uint64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return -1;
  const uint64_t n16 = bytes / 16;
  hipLaunchKernelGGL(calib_read_kernel, dim3(grid_for(n16)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), n16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// On-chip ceiling kernels.  kind: 0 LDS (mode 0-7), 1 vector unit (mode 0-8),
// 2 matrix cores (mode 0-2).  blocks workgroups of 256 threads, iters loop
// iterations of 16 (LDS, vector) or 4 (matrix) operations per lane or wave;
// sink holds blocks * 256 words.  Returns 0, -1 for bad arguments, -3 for a
// launch error.
int loopvq_calib_onchip(int kind, int mode, int blocks, int iters, uint32_t* sink, void* stream) {
  if (!sink || blocks <= 0 || iters <= 0) return -1;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 g(blocks), t(256);
  if (kind == 0) {
    switch (mode) {
      case 0: hipLaunchKernelGGL(calib_lds_kernel<0>, g, t, 0, st, sink, iters); break;
      case 1: hipLaunchKernelGGL(calib_lds_kernel<1>, g, t, 0, st, sink, iters); break;
      case 2: hipLaunchKernelGGL(calib_lds_kernel<2>, g, t, 0, st, sink, iters); break;
      case 3: hipLaunchKernelGGL(calib_lds_kernel<3>, g, t, 0, st, sink, iters); break;
      case 4: hipLaunchKernelGGL(calib_lds_kernel<4>, g, t, 0, st, sink, iters); break;
      case 5: hipLaunchKernelGGL(calib_lds_kernel<5>, g, t, 0, st, sink, iters); break;
      case 6: hipLaunchKernelGGL(calib_lds_kernel<6>, g, t, 0, st, sink, iters); break;
      case 7: hipLaunchKernelGGL(calib_lds_kernel<7>, g, t, 0, st, sink, iters); break;
      default: return -1;
    }
  } else if (kind == 1) {
    switch (mode) {
      case 0: hipLaunchKernelGGL(calib_valu_kernel<0>, g, t, 0, st, sink, iters); break;
      case 1: hipLaunchKernelGGL(calib_valu_kernel<1>, g, t, 0, st, sink, iters); break;
      case 2: hipLaunchKernelGGL(calib_valu_kernel<2>, g, t, 0, st, sink, iters); break;
      case 3: hipLaunchKernelGGL(calib_valu_kernel<3>, g, t, 0, st, sink, iters); break;
      case 4: hipLaunchKernelGGL(calib_valu_kernel<4>, g, t, 0, st, sink, iters); break;
      case 5: hipLaunchKernelGGL(calib_valu_kernel<5>, g, t, 0, st, sink, iters); break;
      case 6: hipLaunchKernelGGL(calib_valu_kernel<6>, g, t, 0, st, sink, iters); break;
      case 7: hipLaunchKernelGGL(calib_valu_kernel<7>, g, t, 0, st, sink, iters); break;
      case 8: hipLaunchKernelGGL(calib_valu_kernel<8>, g, t, 0, st, sink, iters); break;
      default: return -1;
    }
  } else if (kind == 2) {
    switch (mode) {
      case 0: hipLaunchKernelGGL(calib_mfma_kernel<0>, g, t, 0, st, sink, iters); break;
      case 1: hipLaunchKernelGGL(calib_mfma_kernel<1>, g, t, 0, st, sink, iters); break;
      case 2: hipLaunchKernelGGL(calib_mfma_kernel<2>, g, t, 0, st, sink, iters); break;
      default: return -1;
    }
  } else {
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
