// FlashAttention-2 forward for fp32 inputs on gfx950.
//
// Same schedule as the bf16 kernel (a workgroup per 128-row query tile of one
// (batch, head); each of 4 wavefronts owns 32 query rows; K/V tiles shared
// through LDS; running max / denominator in registers; the division once per
// query tile -- Saraf, "FlashAttention 2: Three Places the Chip Was Still
// Waiting", sections 2.2-2.4), but every step stays in fp32:
//   S^T (32 keys x 32 queries) = K_j Q^T  with v_mfma_f32_32x32x2_f32,
//   P in fp32 (no rounding before the second product),
//   O^T (d x 32 queries) += V_j^T P^T     with v_mfma_f32_32x32x2_f32.
// Each k-step of the second product consumes one accumulator element of
// S^T per lane: element i of lane (l32, half) is key 8*(i/4) + 4*half + i%4,
// so the V operand of that step is the V row of that key, read untransposed.

#include "fa2_launch.h"

#include <cmath>
#include <cstdint>

namespace fa2 {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = kF32Waves;
constexpr int kRows = 32;
constexpr int kBr = kF32BlockRows;
constexpr int kBc = kF32BlockCols;
constexpr int kThreads = kWaves * 64;

template <int D>
struct GeoF {
  // K rows padded by 2 floats: lanes (l32, half) reading column 2s+half of
  // row l32 land on bank 2*l32 + half (distinct across the wavefront).
  static constexpr int kStrideK = D + 2;  // floats
  // V rows padded by 8 floats: the two halves of a wavefront read rows 4
  // apart, which then start 32 banks apart.
  static constexpr int kStrideV = D + 8;  // floats
  static constexpr int kOffV = kBc * kStrideK;
  static constexpr int kLdsFloats = kOffV + kBc * kStrideV;
  static constexpr int kChunksPerRow = D / 4;  // float4 chunks
  static constexpr int kRowsPerPass = kThreads / kChunksPerRow;
  static constexpr int kPasses = kBc / kRowsPerPass;
  static constexpr int kKSteps = D / 2;
  static constexpr int kDBlocks = D / 32;
  static_assert(kBc % kRowsPerPass == 0, "tile rows must split evenly");
};

__device__ __forceinline__ float max_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                    const float* __restrict__ v, void* __restrict__ o, float* __restrict__ lse,
                    int BH, int N, int T, float c, float scale, int group) {
  using G = GeoF<D>;
  __shared__ __attribute__((aligned(16))) float smem[G::kLdsFloats];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const int bh = blockIdx.x % BH;
  const int tr = blockIdx.x / BH;
  const int t = CAUSAL ? (T - 1 - tr) : tr;
  const long long head = (long long)bh * N * D;
  // grouped key/value heads: `group` consecutive query heads share one
  const long long kv_head = (long long)(bh / group) * N * D;
  const float* qh = q + head;
  const float* kh = k + kv_head;
  const float* vh = v + kv_head;

  const int q0 = t * kBr;
  const int qw = q0 + wave * kRows;
  const int qrow = qw + l32;

  // Q as B operands: lane (l32, half) holds Q[qrow][2s + half].
  float qf[G::kKSteps];
#pragma unroll
  for (int s = 0; s < G::kKSteps; ++s) qf[s] = (qrow < N) ? qh[(long long)qrow * D + 2 * s + half] : 0.f;

  const int nk = (N + kBc - 1) / kBc;
  int n_tiles = nk;
  if (CAUSAL) {
    const int last_row = min(q0 + kBr - 1, N - 1);
    n_tiles = min(nk, last_row / kBc + 1);
  }

  const int srow = tid / G::kChunksPerRow;
  const int schunk = tid % G::kChunksPerRow;
  float4 kreg[G::kPasses], vreg[G::kPasses];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int key = j * kBc + srow + p * G::kRowsPerPass;
      float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
      if (key < N) {
        kx = *(const float4*)(kh + (long long)key * D + schunk * 4);
        vx = *(const float4*)(vh + (long long)key * D + schunk * 4);
      }
      kreg[p] = kx;
      vreg[p] = vx;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int row = srow + p * G::kRowsPerPass;
      float* kd = smem + row * G::kStrideK + schunk * 4;  // 8-byte aligned
      *(float2*)(kd) = make_float2(kreg[p].x, kreg[p].y);
      *(float2*)(kd + 2) = make_float2(kreg[p].z, kreg[p].w);
      *(float4*)(smem + G::kOffV + row * G::kStrideV + schunk * 4) = vreg[p];
    }
  };

  f32x16 oacc[G::kDBlocks];
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = -1e30f;
  float l = 0.f;

  load_tile(0);
  for (int j = 0; j < n_tiles; ++j) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (j + 1 < n_tiles) load_tile(j + 1);

    const int key0 = j * kBc;
    const bool active = (qw < N) && (!CAUSAL || key0 <= qw + kRows - 1);
    if (!active) continue;

    // S^T = K_j Q^T: lane (l32, half) supplies K[key0 + l32][2s + half].
    f32x16 sacc;
#pragma unroll
    for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
    const float* krow = smem + l32 * G::kStrideK + half;
#pragma unroll
    for (int s = 0; s < G::kKSteps; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * s], qf[s], sacc, 0, 0, 0);

    const bool need_mask = (CAUSAL && key0 + kBc - 1 > qw) || (key0 + kBc > N);
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + 8 * (i >> 2) + 4 * half + (i & 3);
        const bool vis = (key < N) && (!CAUSAL || key <= qrow);
        if (!vis) sacc[i] = -INFINITY;
      }
    }

    float mx = m;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    const float m_new = max_halves(mx);
    const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
    const float mc = m_new * c;
    m = m_new;

    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float s = sacc[i];
      float p = __builtin_amdgcn_exp2f(fmaf(s, c, -mc));
      if (need_mask && s == -INFINITY) p = 0.f;
      rs += p;
      sacc[i] = p;
    }
    l = fmaf(l, alpha, rs);

    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }

    // O^T += V_j^T P^T, one k-step per accumulator element.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float* vrow = smem + G::kOffV + (8 * (i >> 2) + 4 * half + (i & 3)) * G::kStrideV + l32;
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[32 * db], sacc[i], oacc[db], 0, 0, 0);
    }
  }

  const float lt = sum_halves(l);
  if (qrow >= N) return;
  const float inv = 1.0f / lt;
  const long long orow = head + (long long)qrow * D;
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int dcol = 32 * db + 8 * a4 + 4 * half;
      const float x0 = oacc[db][4 * a4 + 0] * inv, x1 = oacc[db][4 * a4 + 1] * inv;
      const float x2 = oacc[db][4 * a4 + 2] * inv, x3 = oacc[db][4 * a4 + 3] * inv;
      if (OUT_BF16) {
        __bf16* op = (__bf16*)o + orow + dcol;
        op[0] = (__bf16)x0; op[1] = (__bf16)x1; op[2] = (__bf16)x2; op[3] = (__bf16)x3;
      } else {
        *(float4*)((float*)o + orow + dcol) = make_float4(x0, x1, x2, x3);
      }
    }
  if (half == 0) lse[(long long)bh * N + qrow] = fmaf(m, scale, logf(lt));
}

template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_t(const FwdArgs& a) {
  const int T = (a.N + kBr - 1) / kBr;
  const long long grid = (long long)T * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  const float c = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, OUT_BF16>), dim3((unsigned)grid), dim3(kThreads), 0,
                     a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v, a.o, a.lse,
                     a.B * a.H, a.N, T, c, a.scale, a.H / a.Hkv);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a) {
  if (a.causal) return a.o_bf16 ? launch_t<D, true, true>(a) : launch_t<D, true, false>(a);
  return a.o_bf16 ? launch_t<D, false, true>(a) : launch_t<D, false, false>(a);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
  switch (a.d) {
    case 64: return launch_d<64>(a);
    case 128: return launch_d<128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa2
