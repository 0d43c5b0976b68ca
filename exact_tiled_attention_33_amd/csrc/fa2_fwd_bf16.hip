// FlashAttention-2 forward for bf16 inputs on gfx950 (MI355X).
//
// One workgroup = one query tile of 128 rows of one (batch, head): the grid
// spans (query tile, batch*head), so a single long head still yields many
// independent workgroups (Saraf, "FlashAttention 2: Three Places the Chip
// Was Still Waiting", section 2.3).  Each of the 4 wavefronts owns 32 query
// rows from the score tile through to the output, so no wavefront ever
// needs another's partial results (same page, section 2.4).  K and V tiles
// of 64 keys are staged in LDS once and read by all four wavefronts.
//
// Per key tile a wavefront computes the transposed score tile
//     S^T (64 keys x 32 queries) = K_j * Q^T
// with v_mfma_f32_32x32x16_bf16, so that each lane holds scores of ONE query
// (lane % 32) for 32 of the 64 keys.  The row max and row sum are then
// in-lane reductions plus a single exchange between the two 32-lane halves
// (v_permlane32_swap).  The probabilities stay in registers in exactly the
// layout the second product needs as its B operand:
//     O^T (d x 32 queries) += V_j^T * P^T
// where the key index (the contraction) is relabelled to match the score
// accumulator, and V^T operands come straight from the row-major V tile in
// LDS through the gfx950 transposing read ds_read_b64_tr_b16.
//
// Online softmax (Saraf section 1 and section 2.2; Mishra, "FlashAttention-2
// and -3: From Algebra to GPU Scheduling", "Keep the unchanged mathematical
// target in view"): per row a running max m (raw score units), a running
// denominator l and an unnormalised accumulator.  With c = scale*log2(e):
//     m'  = max(m, rowmax S)
//     P   = exp2(S*c - m'*c)          (one FMA + one v_exp_f32 per score)
//     l   = exp2((m - m')*c) * l + rowsum P
//     O^T = exp2((m - m')*c) * O^T    (skipped when no row's max moved)
//     O^T += V^T P^T
// and the division by l happens once, when the query tile is finished
// (Saraf section 2.2).  Causal key tiles entirely above the diagonal are
// never loaded or multiplied; only tiles crossing the diagonal (or the
// ragged end of the sequence) are masked.

#include "fa2_launch.h"

#include <cmath>
#include <cstdint>

namespace fa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWaves = kBf16Waves;
constexpr int kRows = 32;               // query rows per wavefront
constexpr int kBr = kBf16BlockRows;     // query rows per workgroup
constexpr int kBc = kBf16BlockCols;     // keys per K/V tile
constexpr int kThreads = kWaves * 64;

template <int D>
struct Geo {
  // K rows are padded by 16 bytes: the 16 lanes of a b128 read phase hit 16
  // distinct 16-byte bank groups.  V rows are padded by 64 bytes: a
  // transposing read touches 4 rows x 64 bytes per half-wave, which then
  // land on disjoint banks.
  static constexpr int kStrideK = D * 2 + 16;
  static constexpr int kStrideV = D * 2 + 64;
  static constexpr int kOffV = kBc * kStrideK;
  static constexpr int kLdsBytes = kOffV + kBc * kStrideV;
  static constexpr int kChunksPerRow = D / 8;   // 16-byte chunks per row
  static constexpr int kRowsPerPass = kThreads / kChunksPerRow;
  static constexpr int kPasses = kBc / kRowsPerPass;
  static constexpr int kKSteps = D / 16;        // k-steps of the score MFMA
  static constexpr int kDBlocks = D / 32;       // 32-row blocks of O^T
  static_assert(kBc % kRowsPerPass == 0, "tile rows must split evenly");
};

__device__ __forceinline__ float max_halves(float x) {
  // permlane32_swap(x, x): first = x[lane % 32], second = x[lane % 32 + 32].
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, void* __restrict__ o, float* __restrict__ lse,
                     int BH, int N, int T, float c, float scale) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) char smem[G::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;   // query column of this lane
  const int half = lane >> 5;  // which 4-key sub-rows of each 8-key group

  // Grid: workgroup -> (batch*head, query tile).  Causal tiles are issued
  // heaviest (latest rows) first.
  const int bh = blockIdx.x % BH;
  const int tr = blockIdx.x / BH;
  const int t = CAUSAL ? (T - 1 - tr) : tr;

  const long long head = (long long)bh * N * D;
  const __bf16* qh = q + head;
  const __bf16* kh = k + head;
  const __bf16* vh = v + head;

  const int q0 = t * kBr;              // first row of the workgroup
  const int qw = q0 + wave * kRows;    // first row of this wavefront
  const int qrow = qw + l32;           // this lane's query row

  // Q rows of the wavefront as MFMA B operands (query = lane % 32,
  // head-dim slice 16*s + 8*half .. +7), held for the whole key loop.
  bf16x8 qf[G::kKSteps];
#pragma unroll
  for (int s = 0; s < G::kKSteps; ++s) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (qrow < N) x = *(const u32x4*)(qh + (long long)qrow * D + 16 * s + 8 * half);
    qf[s] = __builtin_bit_cast(bf16x8, x);
  }

  // Key tiles this workgroup visits: all of them, or (causal) those that
  // start at or below its last row.
  const int nk = (N + kBc - 1) / kBc;
  int n_tiles = nk;
  if (CAUSAL) {
    const int last_row = min(q0 + kBr - 1, N - 1);
    n_tiles = min(nk, last_row / kBc + 1);
  }

  // Register staging of the next K/V tile (global -> VGPR -> LDS).
  const int srow = tid / G::kChunksPerRow;
  const int schunk = tid % G::kChunksPerRow;
  u32x4 kreg[G::kPasses], vreg[G::kPasses];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int key = j * kBc + srow + p * G::kRowsPerPass;
      u32x4 kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
      if (key < N) {
        kx = *(const u32x4*)(kh + (long long)key * D + schunk * 8);
        vx = *(const u32x4*)(vh + (long long)key * D + schunk * 8);
      }
      kreg[p] = kx;
      vreg[p] = vx;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int p = 0; p < G::kPasses; ++p) {
      const int row = srow + p * G::kRowsPerPass;
      *(u32x4*)(smem + row * G::kStrideK + schunk * 16) = kreg[p];
      *(u32x4*)(smem + G::kOffV + row * G::kStrideV + schunk * 16) = vreg[p];
    }
  };

  f32x16 oacc[G::kDBlocks];
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = -1e30f;  // running max of raw scores (finite start: see alpha)
  float l = 0.f;     // running denominator over this lane's keys

  // Per-lane LDS addresses that do not depend on the tile.
  const char* k_lane = smem + l32 * G::kStrideK + 16 * half;
  // Transposing read: lane i of each 16-lane group points at key row
  // (i / 4) of a 4-row slab and dcol 4*(i % 4) of a 16-column slab; lane i
  // then receives the 4 keys of dcol (i) -> an A operand with dcol = lane%32.
  const char* v_lane = smem + G::kOffV + (4 * half + ((lane & 15) >> 2)) * G::kStrideV +
                       (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  load_tile(0);
  for (int j = 0; j < n_tiles; ++j) {
    __syncthreads();  // every wavefront is done with the previous tile
    store_tile();
    __syncthreads();
    if (j + 1 < n_tiles) load_tile(j + 1);  // in flight during the math

    const int key0 = j * kBc;
    const bool active = (qw < N) && (!CAUSAL || key0 <= qw + kRows - 1);
    if (!active) continue;  // wave-uniform: this tile is above all its rows

    // ---- S^T = K_j Q^T (two 32-key blocks) -------------------------------
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
#pragma unroll
      for (int s = 0; s < G::kKSteps; ++s) {
        const bf16x8 a = *(const bf16x8*)(k_lane + kb * 32 * G::kStrideK + 32 * s);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
      }
    }

    // ---- mask (diagonal / ragged tiles only) -------------------------------
    // Accumulator element i of block kb holds key
    //   key0 + 32*kb + 8*(i/4) + 4*half + (i%4)
    const bool need_mask = (CAUSAL && key0 + kBc - 1 > qw) || (key0 + kBc > N);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          const bool vis = (key < N) && (!CAUSAL || key <= qrow);
          if (!vis) sacc[kb][i] = -INFINITY;
        }
    }

    // ---- online softmax ----------------------------------------------------
    float mx = m;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    const float m_new = max_halves(mx);
    // m starts at -1e30 (finite), so alpha is 0 on the first tile for any
    // scale > 0 and exactly 1 for scale == 0, never NaN.
    const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
    const float mc = m_new * c;
    m = m_new;

    bf16x8 pk[2][2];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float s = sacc[kb][i];
        float p = __builtin_amdgcn_exp2f(fmaf(s, c, -mc));
        if (need_mask && s == -INFINITY) p = 0.f;  // also exact when scale == 0
        rs += p;
        pk[kb][i >> 3][i & 7] = (__bf16)p;
      }
    l = fmaf(l, alpha, rs);

    // The correction cannot be deferred (Saraf section 2.2), but it is a
    // no-op for rows whose max did not move; skip it if none did.
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }

    // ---- O^T += V_j^T P^T --------------------------------------------------
    // Key step (kb, h) covers keys 32*kb + 16*h + {0..15}; operand slot u
    // (0..7) of lane (l32, half) is key 8*(u/4) + 4*half + (u%4) in both the
    // P^T B operand (accumulator elements 8h..8h+7) and the V^T A operand.
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const char* p0 = v_lane + (32 * kb + 16 * h) * G::kStrideV + 64 * db;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0);
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0 + 8 * G::kStrideV));
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[kb][h], oacc[db], 0, 0, 0);
        }
  }

  // ---- finalise: one division per row, then O and LSE ----------------------
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
        bf16x4 y = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
        *(u32x2*)((__bf16*)o + orow + dcol) = __builtin_bit_cast(u32x2, y);
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
  const float c = a.scale * 1.4426950408889634f;  // scale * log2(e)
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, OUT_BF16>), dim3((unsigned)grid), dim3(kThreads), 0,
                     a.stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o, a.lse,
                     a.B * a.H, a.N, T, c, a.scale);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdArgs& a) {
  if (a.causal) return a.o_bf16 ? launch_t<D, true, true>(a) : launch_t<D, true, false>(a);
  return a.o_bf16 ? launch_t<D, false, true>(a) : launch_t<D, false, false>(a);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  switch (a.d) {
    case 64: return launch_d<64>(a);
    case 128: return launch_d<128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa2
