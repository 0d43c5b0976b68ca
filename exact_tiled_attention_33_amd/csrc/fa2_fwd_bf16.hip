// FlashAttention-2 forward for bf16 inputs on gfx950 (MI355X).
//
// Work decomposition (Saraf, "FlashAttention 2: Three Places the Chip Was
// Still Waiting", sections 2.3 and 2.4): one workgroup per query tile of 256
// rows of one (batch, head), so even one long head yields many independent
// workgroups; each of its 8 wavefronts owns 32 query rows from the score
// tile through to the output, so no wavefront needs another's partial
// results.  K and V tiles of 64 keys are brought into LDS once per
// workgroup and read by all 8 wavefronts.
//
// Per key tile j a wavefront computes the transposed score tile
//     S^T (64 keys x 32 queries) = K_j * Q^T
// with v_mfma_f32_32x32x16_bf16, so that each lane holds scores of ONE query
// (lane % 32) for 32 of the 64 keys: the row max and row sum are in-lane
// reductions plus one exchange between the two 32-lane halves
// (v_permlane32_swap).  The probabilities stay in registers in the layout the
// second product needs as its B operand:
//     O^T (d x 32 queries) += V_j^T * P^T
// with the key index (the contraction) relabelled to match the score
// accumulator, and the V^T operands read straight from the row-major V tile
// with the gfx950 transposing LDS read ds_read_b64_tr_b16.
//
// Online softmax (Saraf sections 1 and 2.2; Mishra, "FlashAttention-2 and
// -3: From Algebra to GPU Scheduling", "Keep the unchanged mathematical
// target in view"): per row a reference max m (raw score units), a running
// denominator l and an unnormalised accumulator.  With c = scale*log2(e):
//     P   = exp2(S*c - m*c)          (one FMA + one v_exp_f32 per score)
//     l  += rowsum P;  O^T += V^T P^T
// and when a tile's row max exceeds m by more than a threshold, m moves up
// and l and O^T are first multiplied by exp2((m_old - m_new)*c) -- the
// correction that keeps the result exact.  The division by l happens once,
// when the query tile is finished (Saraf section 2.2).  Causal key tiles
// entirely above the diagonal are never loaded or multiplied; only tiles
// crossing the diagonal (or the ragged end of the sequence) are masked.
//
// Schedule on the SIMD (this is where gfx950 differs from the pages' A100
// design): the scalar work of the softmax costs about as many cycles as the
// matrix work of a tile, so the two must overlap.  The 8 wavefronts form two
// groups of 4, and wavefront w shares its SIMD with wavefront w + 4.  Time
// is cut into phases separated by workgroup barriers; group 1 runs one phase
// behind group 0.  In every phase one group is in a matrix phase (S of tile
// j, then O += V P of tile j-1: 32 MFMAs) while the other is in a vector
// phase (mask, row max, correction, exp2, row sum, bf16 packing of tile j),
// so each SIMD always has MFMA and VALU work from different wavefronts.
// K/V tiles are fetched into registers four phases before use, written to
// 2-deep LDS rings two phases later, and read by both groups.

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

constexpr int kWaves = kBf16Waves;      // 8: two groups of 4
constexpr int kGroupWaves = kWaves / 2;
constexpr int kRows = 32;               // query rows per wavefront
constexpr int kBr = kBf16BlockRows;     // query rows per workgroup
constexpr int kBc = kBf16BlockCols;     // keys per K/V tile
constexpr int kThreads = kWaves * 64;
constexpr int kRing = 2;                // K and V tiles resident per ring

template <int D>
struct Geo {
  // K and V tiles are stored unpadded (64 rows x 2*D bytes) with the 16-byte
  // chunks of each row permuted by an XOR swizzle, so that both the tile
  // writes (1 KiB contiguous per wave instruction) and the operand reads are
  // free of bank conflicts:
  //  * K operand reads (b128): 16 lanes of a phase read 16 consecutive rows
  //    at the same logical chunk -> swizzle by row spreads them over 16
  //    distinct 16-byte slots of a 256-byte bank line;
  //  * V transposing reads: a half-wave reads 4 rows x 64 bytes -> swizzle
  //    by (row % 4) moves each row's 4 chunks to a distinct quarter line.
  static constexpr int kRowBytes = D * 2;
  static constexpr int kTileBytes = kBc * kRowBytes;
  static constexpr int kChunks = kRowBytes / 16;           // 16-byte chunks per row
  static constexpr int kRowsPerInst = 1024 / kRowBytes;     // rows per 1 KiB wave write
  static constexpr int kRowsPerWave = kBc / kWaves;         // tile rows each wave loads
  static constexpr int kInstPerWave = kRowsPerWave / kRowsPerInst;
  static constexpr int kKSteps = D / 16;                    // k-steps of the score MFMA
  static constexpr int kDBlocks = D / 32;                   // 32-row blocks of O^T
  static_assert(kRowsPerWave % kRowsPerInst == 0, "tile rows must split evenly");
  __device__ static constexpr int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static constexpr int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
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

// Raw buffer resource over [base, base + bytes): loads past the end return
// zeros, which is how ragged key tiles and query tails are handled without
// branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Max-correction threshold, in log2 units: the reference max of a row is
// only moved (and the accumulator corrected) when a score would exceed it by
// more than this, so probabilities stay <= 2^8.  Any reference value gives
// the same softmax; the threshold only bounds the range of the unnormalised
// terms (Saraf section 2.2: the correction is what keeps the answer exact).
constexpr float kRescaleThreshold = 8.0f;

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, void* __restrict__ o, float* __restrict__ lse,
                     int BH, int N, int T, float c) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kRing * G::kTileBytes];
  char* const lds_k = smem;
  char* const lds_v = smem + kRing * G::kTileBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform values are made explicit so they live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / kGroupWaves;  // 0 or 1 (group 1 runs one phase behind)
  const int gw = wave % kGroupWaves;   // position within the group = SIMD
  const int l32 = lane & 31;           // query column of this lane
  const int half = lane >> 5;          // which 4-key sub-rows of each 8-key group

  // Grid: workgroup -> (batch*head, query tile).  Causal tiles are issued
  // heaviest (latest rows) first.
  const int bh = blockIdx.x % BH;
  const int tr = blockIdx.x / BH;
  const int t = CAUSAL ? (T - 1 - tr) : tr;

  const long long head = (long long)bh * N * D;
  const __bf16* kh = k + head;
  const __bf16* vh = v + head;

  // Rows: the two wavefronts of a SIMD take adjacent 32-row slices, so the
  // causal work of the two groups stays balanced.
  const int q0 = t * kBr;
  const int qw = q0 + 64 * gw + 32 * grp;  // first row of this wavefront
  const int qrow = qw + l32;               // this lane's query row

  // Q rows of the wavefront as MFMA B operands (query = lane % 32,
  // head-dim slice 16*s + 8*half .. +7), held for the whole key loop.
  // Rows past N read as zeros.
  bf16x8 qf[G::kKSteps];
  {
    const int rows = max(0, min(kRows, N - qw));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head + (long long)min(qw, N) * D, rows * D * 2);
#pragma unroll
    for (int s = 0; s < G::kKSteps; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, load16(rq, (l32 * D + 16 * s + 8 * half) * 2));
  }

  // Key tiles: the workgroup streams n_tiles of them; this wavefront computes
  // on the first n_w (causal: those starting at or below its last row) and
  // masks the ones from n_full on (crossing its diagonal, or the ragged end).
  const int nk = (N + kBc - 1) / kBc;
  int n_tiles = nk, n_w = (qw < N) ? nk : 0, n_full = N / kBc;
  if (CAUSAL) {
    n_tiles = min(nk, (min(q0 + kBr, N) - 1) / kBc + 1);
    n_w = (qw < N) ? min(nk, (min(qw + kRows, N) - 1) / kBc + 1) : 0;
    n_full = min(n_full, (qw + 1) / kBc);
  }

  // Tile staging: each wave fetches kInstPerWave x 1 KiB of a K tile and of a
  // V tile into registers, and later writes them to LDS.  Lane -> (row,
  // stored slot); it fetches the logical chunk that the swizzle puts in that
  // slot, so the LDS writes are contiguous.  Keys past N read as zeros.
  const int ld_row = wave * G::kRowsPerWave + lane / G::kChunks;
  const int ld_slot = lane % G::kChunks;
  u32x4 stage_k[G::kInstPerWave], stage_v[G::kInstPerWave];
  auto fetch_tile = [&](const __bf16* src, u32x4 (&dst)[G::kInstPerWave], int j, bool is_k) {
    const int key0 = j * kBc;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (long long)key0 * D, min(kBc, N - key0) * G::kRowBytes);
#pragma unroll
    for (int i = 0; i < G::kInstPerWave; ++i) {
      const int row = ld_row + i * G::kRowsPerInst;
      const int chunk = ld_slot ^ (is_k ? G::swz_k(row) : G::swz_v(row));
      dst[i] = load16(r, row * G::kRowBytes + chunk * 16);
    }
  };
  auto store_tile = [&](const u32x4 (&src)[G::kInstPerWave], char* dst) {
#pragma unroll
    for (int i = 0; i < G::kInstPerWave; ++i)
      *(u32x4*)(dst + (ld_row + i * G::kRowsPerInst) * G::kRowBytes + ld_slot * 16) = src[i];
  };

  // Per-lane LDS offsets.  K operand (kb, s): row 32*kb + l32, logical
  // chunk 2*s + half.  V transposing read for (db, kb, h, u): lane i of each
  // 16-lane group points at key row (i / 4) of a 4-row slab and dcol
  // 4*(i % 4) of a 16-column slab; lane i then receives the 4 keys of one
  // dcol (lane % 32).
  auto k_off = [&](int kb, int s) {
    const int r = 32 * kb + l32;
    return r * G::kRowBytes + (((2 * s + half) ^ G::swz_k(r)) * 16);
  };
  auto v_off = [&](int db, int kb, int h, int u) {
    const int r = 32 * kb + 16 * h + 8 * u + 4 * half + ((lane & 15) >> 2);
    const int chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    return r * G::kRowBytes + ((chunk ^ G::swz_v(r)) * 16) + 8 * (lane & 1);
  };

  f32x16 oacc[G::kDBlocks];
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  f32x16 sacc[2];
  bf16x8 pk[2][2];
  float m = -1e30f;  // reference max of raw scores (finite start)
  float l = 0.f;     // running denominator over this lane's keys

  // ---- matrix phase of tile j: S_j = K_j Q^T, then O^T += V_{j-1}^T P_{j-1}^T
  // No branches here: for tiles past a wavefront's last row the scores are
  // computed but fully masked in the vector phase, so their P is 0.
  // Operands are read from LDS kAhead MFMAs ahead of their use.
  constexpr int kAhead = 4;
  auto scores_mfma = [&](int j) {
    const char* kbuf = lds_k + (j % kRing) * G::kTileBytes;
    // MFMA n uses k-step s = n / 2 of block kb = n % 2 (two independent chains).
    constexpr int kN = 2 * G::kKSteps;
    auto read_k = [&](int n) { return *(const bf16x8*)(kbuf + k_off(n & 1, n >> 1)); };
    bf16x8 ka[kAhead];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) ka[n] = read_k(n);
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const bf16x8 a = ka[n % kAhead];
      if (n + kAhead < kN) ka[n % kAhead] = read_k(n + kAhead);
      sacc[n & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[n >> 1], n < 2 ? f32x16{} : sacc[n & 1], 0, 0, 0);
    }
  };
  auto pv_mfma = [&](int j) {
    // Key step (kb, h) covers keys 32*kb + 16*h + {0..15}; operand slot u
    // of lane (l32, half) is key 8*(u/4) + 4*half + (u%4) in both the P^T
    // operand (accumulator elements 8h..8h+7) and the V^T one.  MFMA n uses
    // key step n / kDBlocks on O^T block n % kDBlocks.
    const char* vbuf = lds_v + (j % kRing) * G::kTileBytes;
    constexpr int kN = 4 * G::kDBlocks;
    auto read_v = [&](int n, bf16x4 (&dst)[2]) {
      const int db = n % G::kDBlocks, kb = (n / G::kDBlocks) >> 1, h = (n / G::kDBlocks) & 1;
      dst[0] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbuf + v_off(db, kb, h, 0)));
      dst[1] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbuf + v_off(db, kb, h, 1)));
    };
    bf16x4 va[kAhead][2];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) read_v(n, va[n]);
#pragma unroll
    for (int n = 0; n < kN; ++n) {
      const bf16x8 a = __builtin_shufflevector(va[n % kAhead][0], va[n % kAhead][1], 0, 1, 2, 3, 4, 5, 6, 7);
      if (n + kAhead < kN) read_v(n + kAhead, va[n % kAhead]);
      const int db = n % G::kDBlocks, ks = n / G::kDBlocks;
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[ks >> 1][ks & 1], oacc[db], 0, 0, 0);
    }
  };
  auto matrix_phase = [&](int j) {
    __builtin_amdgcn_s_setprio(1);
    scores_mfma(j);
    pv_mfma(j - 1);  // P of tile -1 is all zeros
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- vector phase of tile j: mask, row max, correction, P = exp2(...) ----
  auto vector_phase = [&](int j) {
    if (j >= n_full) {
      // element i of block kb holds key key0 + 32*kb + 8*(i/4) + 4*half + (i%4);
      // tiles at or past n_w lie wholly above this wave's rows -> all masked
      const int key0 = j * kBc;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          const bool vis = (key < N) && (!CAUSAL || key <= qrow);
          if (!vis) sacc[kb][i] = -INFINITY;
        }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = max_halves(mx);
    // Move the reference max only when some row would exceed it by more
    // than the threshold; then correct the banked terms.  The first tile
    // always moves it (m starts at -1e30) unless c is vanishingly small,
    // in which case every probability is 1 and m never matters.
    if (__builtin_amdgcn_ballot_w64((mx - m) * c > kRescaleThreshold)) {
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    // Masked scores are -inf and c > 0, so their probability is exactly 0.
    const float mc = m * c;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kb][i], c, -mc));
        rs += p;
        pk[kb][i >> 3][i & 7] = (__bf16)p;
      }
    l += rs;
  };

  // ---- prologue: K_0, K_1, V_0 in LDS; K_2, V_1 staged in registers -------
  fetch_tile(kh, stage_k, 0, true);
  fetch_tile(vh, stage_v, 0, false);
  store_tile(stage_k, lds_k);
  store_tile(stage_v, lds_v);
  if (n_tiles > 1) {
    fetch_tile(kh, stage_k, 1, true);
    store_tile(stage_k, lds_k + G::kTileBytes);
  }
  if (n_tiles > 2) fetch_tile(kh, stage_k, 2, true);
  if (n_tiles > 1) fetch_tile(vh, stage_v, 1, false);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) pk[kb][h][i] = (__bf16)0.f;
  __syncthreads();

  // ---- phases ----------------------------------------------------------------
  // Phase p: group 0 runs the matrix phase of tile p/2 (p even) or the
  // vector phase of tile (p-1)/2 (p odd); group 1 does the same one phase
  // later.  K_j is read in phases 2j and 2j+1, V_j in phases 2j+2 and 2j+3.
  // At phase 2j (j >= 1) the LDS buffers of K_{j-1} and V_{j-2} are free:
  // the staged K_{j+1} and V_j are written into them (first read in phase
  // 2j+2) and K_{j+2}, V_{j+1} are fetched into the staging registers.
  // Each group runs its own straight-line loop; both pass the same number
  // of barriers.
  auto ring = [&](int j) {
    if (j + 1 < n_tiles) store_tile(stage_k, lds_k + ((j + 1) % kRing) * G::kTileBytes);
    store_tile(stage_v, lds_v + (j % kRing) * G::kTileBytes);
    if (j + 2 < n_tiles) fetch_tile(kh, stage_k, j + 2, true);
    if (j + 1 < n_tiles) fetch_tile(vh, stage_v, j + 1, false);
  };
  if (grp == 0) {
    for (int j = 0; j < n_tiles; ++j) {
      if (j >= 1) ring(j);
      matrix_phase(j);
      __syncthreads();
      vector_phase(j);
      __syncthreads();
    }
    __builtin_amdgcn_s_setprio(1);
    pv_mfma(n_tiles - 1);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
    __syncthreads();
  } else {
    __syncthreads();
    matrix_phase(0);
    __syncthreads();
    for (int j = 1; j < n_tiles; ++j) {
      ring(j);
      vector_phase(j - 1);
      __syncthreads();
      matrix_phase(j);
      __syncthreads();
    }
    vector_phase(n_tiles - 1);
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
    pv_mfma(n_tiles - 1);
    __builtin_amdgcn_s_setprio(0);
    __syncthreads();
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
  // LSE = ln(sum exp(scale*S)) = ln2 * (m*c + log2 l), with the same c the
  // probabilities used.
  if (half == 0) lse[(long long)bh * N + qrow] = (m * c + log2f(lt)) * 0.69314718055994531f;
}

template <int D, bool CAUSAL, bool OUT_BF16>
hipError_t launch_t(const FwdArgs& a) {
  const int T = (a.N + kBr - 1) / kBr;
  const long long grid = (long long)T * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  // c = scale * log2(e), kept >= 1e-30 so that masked (-inf) scores give
  // exactly 0 even for scale == 0; any c that small already makes every
  // probability exactly 1 in fp32.
  const float c = fmaxf(a.scale * 1.4426950408889634f, 1e-30f);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, OUT_BF16>), dim3((unsigned)grid), dim3(kThreads), 0,
                     a.stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o, a.lse,
                     a.B * a.H, a.N, T, c);
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
