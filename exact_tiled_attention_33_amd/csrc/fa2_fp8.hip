// FP8 packing for the forward pass with incoherent processing: each row of
// Q (or K) is rotated by R = diag(signs) H / sqrt(d) (H the Sylvester-
// Hadamard matrix), and each (sequence, head) block of rotated rows is
// quantized to OCP E4M3 codes with one fp32 scale (amax / 448).
//
// Source: Mishra, "FlashAttention-2 and -3: From Algebra to GPU
// Scheduling", "Low precision changes numerical error": a shared orthogonal
// mixing transform applied to Q and K before quantization keeps QK^T in
// exact arithmetic and spreads outliers over all coordinates, and block
// scaling sets how much error quantization introduces.
//
// The rotation is computed in fp32 in a fixed order so that the codes are
// reproducible: signs applied (exact), butterfly stages h = 1, 2, ..., d/2
// replacing (a, b) at (i, i + h) of every 2h-block by (a + b, a - b), then
// one multiply by the fp32 constant 1/sqrt(d).  Quantization: inv = 448 /
// amax (correctly rounded), y = clamp(x * inv, -448, 448), code = E4M3(y)
// rounded to nearest even by the hardware conversion.
//
// Two kernels, no atomics: the first writes each 256-row chunk's largest
// |rotated value| to the caller's workspace; the second takes the block's
// maximum over its chunks, recomputes the rotation and writes the codes
// (and, from chunk 0, the scale).  One thread per row; the row lives in
// registers.  HBM-bound and small next to the attention it feeds.

#include <hip/hip_runtime.h>

#include "fa2_launch.h"

namespace fa2 {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPackRows = 256;  // rows (threads) per workgroup

template <int D>
__device__ __forceinline__ void load_rotate(const __bf16* __restrict__ row, const Fp8Signs& sg, bool rotate,
                                            float (&x)[D]) {
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const u32x4 w = *(const u32x4*)(row + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
      x[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
  if (!rotate) return;
#pragma unroll
  for (int i = 0; i < D; ++i)
    if ((sg.bits[i >> 5] >> (i & 31)) & 1u) x[i] = -x[i];
#pragma unroll
  for (int h = 1; h < D; h *= 2)
#pragma unroll
    for (int i = 0; i < D; ++i)
      if ((i & h) == 0) {
        const float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
  constexpr float kInvSqrtD = D == 64 ? 0.125f : (float)0.08838834764831845;  // 1/sqrt(d), fp32
#pragma unroll
  for (int i = 0; i < D; ++i) x[i] = x[i] * kInvSqrtD;
}

template <int D>
__global__ __launch_bounds__(kPackRows) void fp8_amax_kernel(const __bf16* __restrict__ x, int N, int n_chunks,
                                                             Fp8Signs sg, int rotate, float* __restrict__ partial) {
  const int bh = blockIdx.x / n_chunks, chunk = blockIdx.x % n_chunks;
  const int row = chunk * kPackRows + threadIdx.x;
  float amax = 0.f;
  if (row < N) {
    float v[D];
    load_rotate<D>(x + ((long long)bh * N + row) * D, sg, rotate != 0, v);
#pragma unroll
    for (int i = 0; i < D; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  // workgroup maximum (exact whatever the order)
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  __shared__ float wave_max[kPackRows / 64];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = wave_max[0];
#pragma unroll
    for (int w = 1; w < kPackRows / 64; ++w) m = fmaxf(m, wave_max[w]);
    partial[blockIdx.x] = m;
  }
}

template <int D>
__global__ __launch_bounds__(kPackRows) void fp8_quant_kernel(const __bf16* __restrict__ x, int N, int n_chunks,
                                                              Fp8Signs sg, int rotate,
                                                              const float* __restrict__ partial,
                                                              unsigned char* __restrict__ codes,
                                                              float* __restrict__ scales) {
  const int bh = blockIdx.x / n_chunks, chunk = blockIdx.x % n_chunks;
  const int row = chunk * kPackRows + threadIdx.x;
  float amax = 0.f;
  for (int c = 0; c < n_chunks; ++c) amax = fmaxf(amax, partial[(long long)bh * n_chunks + c]);
  if (chunk == 0 && threadIdx.x == 0) scales[bh] = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  if (row >= N) return;
  unsigned char* const out = codes + ((long long)bh * N + row) * D;
  if (!(amax > 0.f)) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) *(u32x4*)(out + 16 * c) = u32x4{0u, 0u, 0u, 0u};
    return;
  }
  const float inv = __fdiv_rn(448.0f, amax);
  float v[D];
  load_rotate<D>(x + ((long long)bh * N + row) * D, sg, rotate != 0, v);
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4 w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float y[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) y[t] = fminf(fmaxf(v[16 * c + 4 * e + t] * inv, -448.0f), 448.0f);
      int p = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      p = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], p, true);
      w[e] = (unsigned)p;
    }
    *(u32x4*)(out + 16 * c) = w;
  }
}

template <int D>
hipError_t launch_pack_d(const Fp8PackArgs& a) {
  const int n_chunks = (a.N + kPackRows - 1) / kPackRows;
  const long long grid = (long long)a.BH * n_chunks;
  if (grid > 0x7fffffffLL || grid < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fp8_amax_kernel<D>), dim3((unsigned)grid), dim3(kPackRows), 0, a.stream,
                     (const __bf16*)a.x, a.N, n_chunks, a.signs, a.rotate ? 1 : 0, a.partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((fp8_quant_kernel<D>), dim3((unsigned)grid), dim3(kPackRows), 0, a.stream,
                     (const __bf16*)a.x, a.N, n_chunks, a.signs, a.rotate ? 1 : 0, (const float*)a.partial,
                     (unsigned char*)a.codes, a.scales);
  return hipGetLastError();
}

}  // namespace

int fp8_pack_chunks(int N) { return (N + kPackRows - 1) / kPackRows; }

hipError_t launch_fp8_pack(const Fp8PackArgs& a) {
  switch (a.d) {
    case 64: return launch_pack_d<64>(a);
    case 128: return launch_pack_d<128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa2
