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
// (and, from chunk 0, the scale).  A row is a quad of lanes: lane p of the
// quad holds the 16-byte pieces at elements 32k + 8p (k < d/32), so the
// butterfly stages h = 8 and 16 pair lanes of the quad (a DPP move) and all
// other stages pair elements inside a lane, on the same fp32 operands in
// the same order.  HBM-bound and small next to the attention it feeds.

#include <hip/hip_runtime.h>

#include "fa2_launch.h"

namespace fa2 {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPackRows = 256;  // rows per workgroup (a chunk): 64 per wavefront
constexpr int kPackUnroll = 2;  // row groups of a wavefront loaded together

template <int D>
struct PackGeo {
  static constexpr int kK = D / 32;              // 16-byte pieces per lane
  static constexpr int kE = 8 * kK;              // elements per lane
  static constexpr int kGroups = 64 / 16;        // row groups of 16 rows per wavefront
};

// the partner lane's value of the quad: p ^ 1 (xl = 1) or p ^ 2 (xl = 2)
__device__ __forceinline__ float quad_xor(float v, int xl) {
  const int b = __float_as_int(v);
  const int r = xl == 1 ? __builtin_amdgcn_update_dpp(b, b, 0xB1, 0xF, 0xF, false)   // quad_perm [1,0,3,2]
                        : __builtin_amdgcn_update_dpp(b, b, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  return __int_as_float(r);
}

// x[8k + t] = element 32k + 8p + t of the row, rotated in place.  All four
// lanes of the quad must be active.
template <int D>
__device__ __forceinline__ void rotate_quad(const Fp8Signs& sg, bool rotate, int p, float (&x)[PackGeo<D>::kE]) {
  constexpr int kK = PackGeo<D>::kK;
  if (!rotate) return;
#pragma unroll
  for (int k = 0; k < kK; ++k)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int i = 32 * k + 8 * p + t;
      if ((sg.bits[i >> 5] >> (i & 31)) & 1u) x[8 * k + t] = -x[8 * k + t];
    }
  // h = 1, 2, 4: inside each 8-element piece
#pragma unroll
  for (int h = 1; h < 8; h *= 2)
#pragma unroll
    for (int k = 0; k < kK; ++k)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if ((t & h) == 0) {
          const float a = x[8 * k + t], b = x[8 * k + t + h];
          x[8 * k + t] = a + b;
          x[8 * k + t + h] = a - b;
        }
  // h = 8, 16: between the lanes of the quad (element i in lane p, i + h in p ^ h/8)
#pragma unroll
  for (int xl = 1; xl < 4; xl *= 2) {
    const bool upper = (p & xl) != 0;
#pragma unroll
    for (int e = 0; e < 8 * kK; ++e) {
      const float q = quad_xor(x[e], xl);
      x[e] = upper ? q - x[e] : x[e] + q;
    }
  }
  // h = 32, 64: between the pieces of a lane
#pragma unroll
  for (int hk = 1; hk < kK; hk *= 2)
#pragma unroll
    for (int k = 0; k < kK; ++k)
      if ((k & hk) == 0)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float a = x[8 * k + t], b = x[8 * (k + hk) + t];
          x[8 * k + t] = a + b;
          x[8 * (k + hk) + t] = a - b;
        }
  constexpr float kInvSqrtD = D == 64 ? 0.125f : (float)0.08838834764831845;  // 1/sqrt(d), fp32
#pragma unroll
  for (int e = 0; e < 8 * kK; ++e) x[e] = x[e] * kInvSqrtD;
}

// this lane's row in row group g of its wavefront, and its loads (rows
// past N are clamped to N - 1 and not used)
template <int D>
__device__ __forceinline__ void load_quad(const __bf16* __restrict__ xb, int row, int N, float (&x)[PackGeo<D>::kE]) {
  const __bf16* const r = xb + (long long)min(row, N - 1) * D;
#pragma unroll
  for (int k = 0; k < PackGeo<D>::kK; ++k) {
    const u32x4 w = *(const u32x4*)(r + 32 * k);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[8 * k + 2 * e] = __uint_as_float(w[e] << 16);
      x[8 * k + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kPackRows) void fp8_amax_kernel(const __bf16* __restrict__ x, int N, int n_chunks,
                                                             Fp8Signs sg, int rotate, float* __restrict__ partial) {
  using PG = PackGeo<D>;
  const int bh = blockIdx.x / n_chunks, chunk = blockIdx.x % n_chunks;
  const int lane = threadIdx.x & 63, p = lane & 3;
  const int row0 = chunk * kPackRows + (threadIdx.x >> 6) * 64 + (lane >> 2);
  const __bf16* const xb = x + (long long)bh * N * D + 8 * p;
  float amax = 0.f;
  for (int g0 = 0; g0 < PG::kGroups; g0 += kPackUnroll) {
    float v[kPackUnroll][PG::kE];
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u) load_quad<D>(xb, row0 + 16 * (g0 + u), N, v[u]);
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u) {
      rotate_quad<D>(sg, rotate != 0, p, v[u]);
      if (row0 + 16 * (g0 + u) < N)
#pragma unroll
        for (int e = 0; e < PG::kE; ++e) amax = fmaxf(amax, fabsf(v[u][e]));
    }
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
  using PG = PackGeo<D>;
  const int bh = blockIdx.x / n_chunks, chunk = blockIdx.x % n_chunks;
  float amax = 0.f;
  for (int c = 0; c < n_chunks; ++c) amax = fmaxf(amax, partial[(long long)bh * n_chunks + c]);
  if (chunk == 0 && threadIdx.x == 0) scales[bh] = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  const int lane = threadIdx.x & 63, p = lane & 3;
  const int row0 = chunk * kPackRows + (threadIdx.x >> 6) * 64 + (lane >> 2);
  const __bf16* const xb = x + (long long)bh * N * D + 8 * p;
  unsigned char* const ob = codes + (long long)bh * N * D + 8 * p;
  const bool zero = !(amax > 0.f);
  const float inv = zero ? 0.f : __fdiv_rn(448.0f, amax);
  for (int g0 = 0; g0 < PG::kGroups; g0 += kPackUnroll) {
    float v[kPackUnroll][PG::kE];
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u) load_quad<D>(xb, row0 + 16 * (g0 + u), N, v[u]);
#pragma unroll
    for (int u = 0; u < kPackUnroll; ++u) {
      rotate_quad<D>(sg, rotate != 0, p, v[u]);
      const int row = row0 + 16 * (g0 + u);
#pragma unroll
      for (int k = 0; k < PG::kK; ++k) {
        u32x2 cw = {0u, 0u};
        if (!zero) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            float y[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) y[t] = fminf(fmaxf(v[u][8 * k + 4 * e + t] * inv, -448.0f), 448.0f);
            int q = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
            q = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], q, true);
            cw[e] = (unsigned)q;
          }
        }
        if (row < N) *(u32x2*)(ob + (long long)row * D + 32 * k) = cw;
      }
    }
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
