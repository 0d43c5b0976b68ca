// Backward pass of exact attention for bf16 inputs on gfx950 (MI355X).
//
// The gradient of the forward operation (fa2_fwd) given dO, with P
// recomputed from Q, K and the forward's per-row logsumexp instead of being
// stored (Mishra, "FlashAttention-2 and -3: From Algebra to GPU
// Scheduling": a fast kernel may redo arithmetic to avoid moving data; the
// pages name the backward pass as part of the training runs, Saraf,
// "FlashAttention 2: Three Places the Chip Was Still Waiting", section 2.5):
//
//   P_ij  = exp2(S_ij*c - LSE_i*log2(e)),  c = scale*log2(e)
//   D_i   = dO_i . O_i
//   dV_j  = sum_i P_ij dO_i
//   dS_ij = P_ij (dO_i . v_j - D_i)
//   dQ_i  = scale * sum_j dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i
//
// Three kernels, in stream order:
//  * bwd_delta: D for every row (reads dO and O once).
//  * bwd_dkdv: one workgroup per 128-key tile of one (batch, head); each
//    wavefront owns 32 keys and keeps their dK^T and dV^T in registers while
//    32-query blocks of Q and dO stream through LDS.  The 8 wavefronts form
//    two groups of 4 that take alternate query blocks; their partial sums
//    are added through LDS at the end.  With the key on the lane (the N side
//    of the MFMA), S and dP come out as [query x key] accumulators whose
//    registers run over queries, which is exactly the operand layout the
//    dV^T += dO^T P and dK^T += Q^T dS products need for P and dS (the query
//    index of the contraction is relabelled to match).
//  * bwd_dq: one workgroup per 256-query tile (8 wavefronts x 32 queries, as
//    in the forward kernel); 64-key tiles of K and V stream through LDS;
//    S^T and dP^T are [key x query] with the query on the lane, and
//    dQ^T += K^T dS^T consumes dS^T in the same relabelled layout.
// No atomics: every output element is written by exactly one wavefront.
//
// LDS tiles hold rows of 2*d bytes (d = 64 or 128) with no padding.  A
// tile is read both along rows (16-byte operand reads: 16 lanes, 16 rows,
// one column) and across rows (ds_read_b64_tr_b16: 4 consecutive rows of a
// 64-byte column block), so instead of padding, the 16-byte chunk c of row
// r is stored at position c ^ swz(r) (BG below): the 16 rows of a row read
// land on 16 distinct 16-byte slots and the 4 rows of a transposing read on
// 4 distinct 64-byte quarters of the 256-byte bank line, so both are free
// of bank conflicts.  The permutation is applied on
// the global side of the global->LDS copies (each lane fetches the chunk
// that belongs at its LDS slot).

#include "fa2_launch.h"

#include <cmath>
#include <cstdint>
#include <type_traits>

namespace fa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLog2e = 1.4426950408889634f;

// Geometry of head dimension D (64 or 128): LDS rows of 2*D bytes (no
// padding), the k-steps of a d-contraction MFMA and the 32-row blocks of a
// d-sized accumulator.  The 16-byte chunk c of row r sits at position
// c ^ swz(r).  D = 128 (16 chunks, one row per 256-byte bank line):
// swz(r) = 4*(r%4) + (r/4)%4.  D = 64 (8 chunks, two rows per bank line):
// swz(r) = (r/4)%4 + 4*((r/2)%2), which puts the 16 rows of a row-read
// phase on the 16 distinct 16-byte slots of the bank line and the 4 rows of
// a transposing read on its 4 distinct 64-byte quarters.
template <int D>
struct BG {
  static_assert(D == 64 || D == 128, "head dimension 64 or 128");
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks per row
  static constexpr int kRowsPerCopy = 1024 / kRowBytes;  // rows per 64-lane x 16-byte copy
  static constexpr int kKSteps = D / 16;
  static constexpr int kDBlocks = D / 32;
  static __device__ __forceinline__ int swz(int r) {
    return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : (((r >> 2) & 3) | (((r >> 1) & 1) << 2));
  }
};

template <typename T>
__device__ __forceinline__ T pin(T x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Buffer descriptor in scalar registers (wave-uniform base and size; loads
// past `bytes` return zeros).
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, int bytes) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  i32x4 r = {__builtin_amdgcn_readfirstlane((int)(b & 0xffffffffu)),
             __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xffffu)),
             __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
  return r;
}

// Global -> LDS copies: lane i's 16 (resp. 4) bytes from byte offset voff
// of the buffer land at LDS byte offset lds_offset + 16*i (resp. 4*i).
// Inline assembly keeps the compiler from treating later LDS reads as
// dependent on the copy; completion is tracked with wait_vmem and published
// with a workgroup barrier.  Clobbers m0, which nothing else here uses.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, int voff, unsigned lds_offset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_offset), "v"(voff), "s"(rsrc) : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(i32x4 rsrc, int voff, unsigned lds_offset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds_offset), "v"(voff), "s"(rsrc) : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ unsigned lds_offset_of(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// s_waitcnt: at most n vector-memory operations of this wave outstanding.
__device__ __forceinline__ void wait_vmem(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F74); break;
  }
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Per-lane LDS offsets within a swizzled tile.
//  row(s):    the 16-byte operand read of row l32 (+ multiples of 32 rows),
//             k-step s, i.e. columns 16*s + 8*half .. +7;
//  tr(db, u): the transposing read of rows 4*half + (lane%16)/4 (+ 8*u +
//             multiples of 16 rows) in 64-byte column block db: lane i of
//             each 16-lane group points at row i/4 of a 4-row slab and at
//             columns 4*(i%4) .. +3 of a 16-column slab.
template <int D>
struct LdsOffsets {
  int row[BG<D>::kKSteps];
  int tr[BG<D>::kDBlocks][2];
};

template <int D>
__device__ __forceinline__ LdsOffsets<D> lds_offsets(int lane) {
  using Gm = BG<D>;
  LdsOffsets<D> o;
  const int l32 = lane & 31, half = lane >> 5;
  const int sw = Gm::swz(l32);
#pragma unroll
  for (int s = 0; s < Gm::kKSteps; ++s) o.row[s] = l32 * Gm::kRowBytes + 16 * ((2 * s + half) ^ sw);
  const int t4 = (lane & 15) >> 2;                          // row within the 4-row slab
  const int e = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // 16-byte chunk within the 64-byte block
  // the slab's rows r = 4*half + t4 (+ 8u): their 64-byte block db sits at
  // db ^ (bits 2-3 of swz(r)), the chunk within it at e ^ (bits 0-1)
  const int bq = D == 128 ? t4 : (t4 >> 1);
#pragma unroll
  for (int db = 0; db < Gm::kDBlocks; ++db)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      o.tr[db][u] = (4 * half + t4) * Gm::kRowBytes + 64 * (db ^ bq) + 16 * (e ^ (half + 2 * u)) + 8 * (lane & 1);
  return o;
}

// Source byte offset (relative to the tile's first row) of the chunk that a
// lane of copy instruction i puts into LDS: instruction i fills rows
// kRowsPerCopy*i .. +kRowsPerCopy-1 (64 lanes x 16 bytes, in LDS order).
template <int D>
__device__ __forceinline__ int copy_voff(int lane, int i) {
  using Gm = BG<D>;
  const int r = Gm::kRowsPerCopy * i + lane / Gm::kChunks;
  return r * Gm::kRowBytes + 16 * ((lane % Gm::kChunks) ^ Gm::swz(r));
}

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i: D/8 lanes per row, 8 elements per lane.
template <int D, bool O_BF16>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const void* __restrict__ o, const __bf16* __restrict__ dout,
                                                        float* __restrict__ delta, long long rows) {
  constexpr int kLanes = D / 8;  // lanes per row
  const long long row = (long long)blockIdx.x * (256 / kLanes) + (threadIdx.x / kLanes);
  const int part = threadIdx.x % kLanes;
  float acc = 0.f;
  if (row < rows) {
    const long long base = row * D + part * 8;
    const bf16x8 g = *(const bf16x8*)(dout + base);
    float ov[8];
    if (O_BF16) {
      const bf16x8 x = *(const bf16x8*)((const __bf16*)o + base);
#pragma unroll
      for (int i = 0; i < 8; ++i) ov[i] = (float)x[i];
    } else {
      const f32x4 x0 = *(const f32x4*)((const float*)o + base);
      const f32x4 x1 = *(const f32x4*)((const float*)o + base + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) { ov[i] = x0[i]; ov[4 + i] = x1[i]; }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = fmaf((float)g[i], ov[i], acc);
  }
#pragma unroll
  for (int m = kLanes / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, kLanes);
  if (row < rows && part == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK and dV.  Grid: blockIdx.x = key tile * B*Hkv + key/value head (key tiles in ascending
// order: under a causal mask the first tiles see the most queries).
constexpr int kKVWaves = 8;
constexpr int kKVKeys = kBwdKVKeys;                    // 128 = 4 waves x 32 keys
constexpr int kQB = kBwdKVRows;                        // 32 queries per block
template <int D>
struct KVG {
  static constexpr int kKVTileBytes = kKVKeys * BG<D>::kRowBytes;  // K or V tile: 32 KiB at d = 128
  static constexpr int kQBBytes = kQB * BG<D>::kRowBytes;          // Q or dO block: 8 KiB at d = 128
  static constexpr int kSlotBytes = 2 * kQBBytes + 2 * 256;        // Q, dO, LSE row, D row
  static constexpr int kLds = 2 * kKVTileBytes + 4 * kSlotBytes;   // 2 groups x 2 slots
  static constexpr int kAccVals = 2 * BG<D>::kDBlocks * 16;        // dV and dK values per lane
  static_assert(kLds >= 4 * kAccVals * 64 * 4, "partial sums of one group must fit in LDS");
};

template <int D, bool MASKED, bool GRAD_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(kKVWaves * 64, kKVWaves * 64), amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                     const __bf16* __restrict__ dout, const float* __restrict__ lse,
                     const float* __restrict__ delta, void* __restrict__ dk, void* __restrict__ dv,
                     int BHkv, int N, float c, float scale, int group, int wl, int wr) {
  using Gm = BG<D>;
  constexpr int kD = D, kRowBytes = Gm::kRowBytes, kKSteps = Gm::kKSteps, kDBlocks = Gm::kDBlocks;
  constexpr int kKVTileBytes = KVG<D>::kKVTileBytes, kQBBytes = KVG<D>::kQBBytes;
  constexpr int kSlotBytes = KVG<D>::kSlotBytes, kAccVals = KVG<D>::kAccVals;
  __shared__ __attribute__((aligned(1024))) char smem[KVG<D>::kLds];
  const char* const lds_k = smem;
  const char* const lds_v = smem + kKVTileBytes;
  char* const lds_ring = smem + 2 * kKVTileBytes;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;  // query blocks b with b % 2 == grp (relative to the first)
  const int gw = wave & 3;    // keys 32*gw .. +31 of the tile
  const int l32 = lane & 31, half = lane >> 5;

  // Grid: key/value head bkv, key tile kt.  With grouped heads the `group`
  // query heads bkv*group .. bkv*group + group-1 all read this head, and its
  // dK, dV sum over them: the query blocks of every one of them are
  // streamed through the same accumulators.
  const int bkv = blockIdx.x % BHkv;
  const int kt = blockIdx.x / BHkv;
  const int k0 = kt * kKVKeys;
  const long long head = (long long)bkv * N * kD;  // K, V, dK, dV
  const int kw0 = k0 + 32 * gw;  // first key of this wave
  const int key = kw0 + l32;     // this lane's key
  // Key j is visible to query i iff i - wl <= j <= i + wr (-1: no limit on
  // that side; causal: wl = -1, wr = 0).  This lane's key is seen by the
  // queries [q_lo, q_hi] (empty past N): the mask is two compares.
  const int q_lo = (MASKED && wr >= 0) ? max(0, key - wr) : 0;
  const int q_hi = key >= N ? -1 : ((MASKED && wl >= 0) ? min(N - 1, key + wl) : N - 1);

  // ---- K and V tiles (once): kKVKeys / kRowsPerCopy copy instructions each ----
  {
    const int rows = min(kKVKeys, N - k0);
    const i32x4 rk = raw_rsrc(k + head + (long long)k0 * kD, rows * kRowBytes);
    const i32x4 rv = raw_rsrc(v + head + (long long)k0 * kD, rows * kRowBytes);
    const unsigned base = __builtin_amdgcn_readfirstlane(lds_offset_of(smem));
#pragma unroll
    for (int m = 0; m < kKVKeys / Gm::kRowsPerCopy / kKVWaves; ++m) {
      const int i = wave + kKVWaves * m;
      copy16_to_lds(rk, copy_voff<D>(lane, i), base + 1024 * i);
      copy16_to_lds(rv, copy_voff<D>(lane, i), base + kKVTileBytes + 1024 * i);
    }
  }

  // ---- query blocks ----
  // The work is the list of (query head, block) pairs, query head major;
  // step s of wave group grp takes item 2s + grp.
  const int nqb = (N + kQB - 1) / kQB;
  // query blocks holding a query that sees a key of this tile
  const int b_first = (MASKED && wr >= 0) ? max(0, k0 - wr) / kQB : 0;
  const int b_last = (MASKED && wl >= 0) ? min(N - 1, min(k0 + kKVKeys, N) - 1 + wl) / kQB : nqb - 1;
  const int nb = b_last - b_first + 1;  // blocks per query head
  const int n_items = group * nb;
  const int n_steps = (n_items + 1) / 2;
  // group-local copy of item it into ring slot `slot`: Q and dO
  // kQB / kRowsPerCopy instructions each, then the LSE and D rows.
  auto copy_block = [&](int it, int slot) __attribute__((always_inline)) {
    const int hq = bkv * group + it / nb;  // query head
    const int q0 = (b_first + it % nb) * kQB;
    const long long qhead = (long long)hq * N * kD;
    const int rows = max(0, min(kQB, N - q0));
    const i32x4 rq = raw_rsrc(q + qhead + (long long)q0 * kD, rows * kRowBytes);
    const i32x4 rg = raw_rsrc(dout + qhead + (long long)q0 * kD, rows * kRowBytes);
    const unsigned base =
        __builtin_amdgcn_readfirstlane(lds_offset_of(lds_ring)) + (unsigned)((grp * 2 + slot) * kSlotBytes);
#pragma unroll
    for (int m = 0; m < kQB / Gm::kRowsPerCopy / 4; ++m) {
      const int i = gw + 4 * m;
      copy16_to_lds(rq, copy_voff<D>(lane, i), base + 1024 * i);
      copy16_to_lds(rg, copy_voff<D>(lane, i), base + kQBBytes + 1024 * i);
    }
    if (gw < 2) {
      const float* src = (gw == 0 ? lse : delta) + (long long)hq * N + q0;
      copy4_to_lds(raw_rsrc(src, rows * 4), 4 * lane, base + 2 * kQBBytes + 256 * gw);
    }
  };

  f32x16 dvacc[kDBlocks], dkacc[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dvacc[db][i] = 0.f; dkacc[db][i] = 0.f; }

  // Per-lane LDS offsets, fixed for the whole kernel: the wave's 32 rows of
  // the K and V tiles (row reads), and its group's ring slot 0 (row and
  // transposing reads); slot 1 and the dO block are immediates on top.
  int krw[kKSteps], qrw[kKSteps], qtr[kDBlocks][2];
  {
    const LdsOffsets<D> off = lds_offsets<D>(lane);
    const int ring = 2 * kKVTileBytes + grp * 2 * kSlotBytes;
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      krw[s] = off.row[s] + 32 * gw * kRowBytes;
      qrw[s] = off.row[s] + ring;
    }
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u) qtr[db][u] = off.tr[db][u] + ring;
  }

  auto compute = [&](int b, auto slot_c) __attribute__((always_inline)) {
    constexpr int kSlot = decltype(slot_c)::value * kSlotBytes;
    const int q0 = b * kQB;
    const float* const slse = (const float*)(lds_ring + (grp * 2 + decltype(slot_c)::value) * kSlotBytes + 2 * kQBBytes);
    const float* const sdel = slse + 64;

    // S = Q K^T and dP = dO V^T, [32 queries x 32 keys]: the key is the
    // lane (l32); element i holds query q0 + 8*(i/4) + 4*half + (i%4).
    f32x16 sacc = {}, dpacc = {};
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      const bf16x8 qa = *(const bf16x8*)(smem + qrw[s] + kSlot);
      const bf16x8 kb = *(const bf16x8*)(lds_k + krw[s]);
      sacc = mfma(qa, kb, sacc);
    }
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      const bf16x8 ga = *(const bf16x8*)(smem + qrw[s] + kSlot + kQBBytes);
      const bf16x8 vb = *(const bf16x8*)(lds_v + krw[s]);
      dpacc = mfma(ga, vb, dpacc);
    }
    // P and dS.  Blocks not wholly inside every key's band (and ragged
    // edges) are masked (P = 0).
    const bool edge = (MASKED && ((wr >= 0 && q0 < kw0 + 31 - wr) || (wl >= 0 && q0 + 31 > kw0 + wl))) ||
                      q0 + kQB > N || kw0 + 32 > N;
    if (edge) {
      // a real branch: blocks inside every key's band skip the mask (the
      // empty volatile statement keeps the compiler from applying it to
      // every block as selects)
      asm volatile("");
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qq = q0 + 8 * (i >> 2) + 4 * half + (i & 3);
        sacc[i] = (qq >= q_lo) & (qq <= q_hi) ? sacc[i] : -INFINITY;
      }
    }
    float p[16], ds[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l4 = *(const f32x4*)(slse + 8 * g + 4 * half);
      const f32x4 d4 = *(const f32x4*)(sdel + 8 * g + 4 * half);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        const float pi = __builtin_amdgcn_exp2f(fmaf(sacc[i], c, -l4[r] * kLog2e));
        p[i] = pi;
        ds[i] = pi * (dpacc[i] - d4[r]);
      }
    }
    // bf16 operands: slot u of lane (key, half) in step h is query
    // 16*h + 8*(u/4) + 4*half + (u%4), i.e. elements 8h .. 8h+7.
    bf16x8 pk[2], dsk[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        pk[h][u] = (__bf16)p[8 * h + u];
        dsk[h][u] = (__bf16)ds[8 * h + u];
      }
    // dV^T += dO^T P and dK^T += Q^T dS, [d x keys]: A operands by
    // transposing reads of the dO and Q blocks.
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + qtr[db][0] + kSlot + kQBBytes + 16 * h * kRowBytes));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + qtr[db][1] + kSlot + kQBBytes + (16 * h + 8) * kRowBytes));
        dvacc[db] = mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pk[h], dvacc[db]);
      }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) {
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + qtr[db][0] + kSlot + 16 * h * kRowBytes));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + qtr[db][1] + kSlot + (16 * h + 8) * kRowBytes));
        dkacc[db] = mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), dsk[h], dkacc[db]);
      }
  };

  // Prologue: K, V and each group's first item in LDS.
  if (grp < n_items) copy_block(grp, 0);
  wait_vmem(0);
  __syncthreads();
  // Step s: this group's item 2s + grp from ring slot s % 2, while the item
  // of step s+1 is copied into the other slot (last read in step s-1, which
  // every wave finished before the barrier that ended it).
  auto step = [&](int s, auto slot_c) __attribute__((always_inline)) {
    constexpr int kSl = decltype(slot_c)::value;
    const int it = 2 * s + grp;
    if (it + 2 < n_items) copy_block(it + 2, kSl ^ 1);
    const int b = b_first + it % nb;
    // a block with no query that sees one of this wave's keys contributes 0
    const bool outside = MASKED && ((wr >= 0 && b * kQB + kQB - 1 < kw0 - wr) ||
                                    (wl >= 0 && b * kQB > kw0 + 31 + wl));
    if (it < n_items && !outside) compute(b, slot_c);
    wait_vmem(0);
    __syncthreads();
  };
  using Sl0 = std::integral_constant<int, 0>;
  using Sl1 = std::integral_constant<int, 1>;
  int s = 0;
  for (; s + 1 < n_steps; s += 2) {
    step(s, Sl0{});
    step(s + 1, Sl1{});
  }
  if (s < n_steps) step(s, Sl0{});

  // ---- add the two groups' partial sums, then store ----
  float* const red = (float*)smem;  // [wave 0..3][kAccVals values][64 lanes]
  if (grp == 1) {
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        red[((gw * kAccVals) + db * 16 + i) * 64 + lane] = dvacc[db][i];
        red[((gw * kAccVals) + kAccVals / 2 + db * 16 + i) * 64 + lane] = dkacc[db][i];
      }
  }
  __syncthreads();
  if (grp == 1 || key >= N) return;
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dvacc[db][i] += red[((gw * kAccVals) + db * 16 + i) * 64 + lane];
      dkacc[db][i] = (dkacc[db][i] + red[((gw * kAccVals) + kAccVals / 2 + db * 16 + i) * 64 + lane]) * scale;
    }
  const long long krow = head + (long long)key * kD;
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int dcol = 32 * db + 8 * a4 + 4 * half;
      if (GRAD_BF16) {
        const bf16x4 yv = {(__bf16)dvacc[db][4 * a4], (__bf16)dvacc[db][4 * a4 + 1], (__bf16)dvacc[db][4 * a4 + 2], (__bf16)dvacc[db][4 * a4 + 3]};
        const bf16x4 yk = {(__bf16)dkacc[db][4 * a4], (__bf16)dkacc[db][4 * a4 + 1], (__bf16)dkacc[db][4 * a4 + 2], (__bf16)dkacc[db][4 * a4 + 3]};
        *(u32x2*)((__bf16*)dv + krow + dcol) = __builtin_bit_cast(u32x2, yv);
        *(u32x2*)((__bf16*)dk + krow + dcol) = __builtin_bit_cast(u32x2, yk);
      } else {
        *(float4*)((float*)dv + krow + dcol) = make_float4(dvacc[db][4 * a4], dvacc[db][4 * a4 + 1], dvacc[db][4 * a4 + 2], dvacc[db][4 * a4 + 3]);
        *(float4*)((float*)dk + krow + dcol) = make_float4(dkacc[db][4 * a4], dkacc[db][4 * a4 + 1], dkacc[db][4 * a4 + 2], dkacc[db][4 * a4 + 3]);
      }
    }
}

// ---------------------------------------------------------------------------
// dQ.  Grid: blockIdx.x = query tile * BH + bh (causal: heaviest first).
constexpr int kQWaves = kBwdQWaves;             // 8
constexpr int kQRows = kBwdQRows;               // 256
constexpr int kQCols = kBwdQCols;               // 64 keys per tile
constexpr int kQRing = 3;

template <int D, bool MASKED, bool GRAD_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(kQWaves * 64, kQWaves * 64), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
                   const __bf16* __restrict__ dout, const float* __restrict__ lse,
                   const float* __restrict__ delta, void* __restrict__ dq, int BH, int N, int T, float c,
                   float scale, int group, int wl, int wr) {
  using Gm = BG<D>;
  constexpr int kD = D, kRowBytes = Gm::kRowBytes, kKSteps = Gm::kKSteps, kDBlocks = Gm::kDBlocks;
  constexpr int kQTileBytes = kQCols * kRowBytes;  // K or V tile: 16 KiB at d = 128
  constexpr int kQStage = 2 * kQTileBytes;         // K then V
  __shared__ __attribute__((aligned(1024))) char smem[kQRing * kQStage];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, half = lane >> 5;

  const int bh = blockIdx.x % BH;
  const int tr = blockIdx.x / BH;
  const int t = MASKED ? (T - 1 - tr) : tr;
  const long long head = (long long)bh * N * kD;
  // grouped key/value heads: `group` consecutive query heads share one
  const long long kv_head = (long long)(bh / group) * N * kD;
  const int q0 = t * kQRows;
  const int qw = q0 + 32 * wave;
  const int qrow = qw + l32;

  // Q and dO rows of the wavefront as MFMA B operands (query = lane % 32,
  // columns 16*s + 8*half .. +7); rows past N read as zeros.
  bf16x8 qf[kKSteps], gf[kKSteps];
  {
    const int rows = max(0, min(32, N - qw));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head + (long long)min(qw, N) * kD, rows * kRowBytes);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(dout + head + (long long)min(qw, N) * kD, rows * kRowBytes);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8, load16(rq, (l32 * kD + 16 * s + 8 * half) * 2));
      gf[s] = __builtin_bit_cast(bf16x8, load16(rg, (l32 * kD + 16 * s + 8 * half) * 2));
    }
  }
  const float nlse2 = qrow < N ? -lse[(long long)bh * N + qrow] * kLog2e : 0.f;
  const float dlt = qrow < N ? delta[(long long)bh * N + qrow] : 0.f;

  // Key tiles streamed: j_lo .. j_lo + n_tiles - 1 (those with a key some
  // row of the workgroup sees); this wavefront computes on jw_lo .. jw_hi-1
  // and needs no mask on jf_lo .. jf_hi-1 (keys below N that all its rows
  // see).  Key j is visible to query i iff i - wl <= j <= i + wr.
  const int nk = (N + kQCols - 1) / kQCols;
  int j_lo = 0, n_tiles = nk, jw_lo = 0, jw_hi = (qw < N) ? nk : 0, jf_lo = 0, jf_hi = N / kQCols;
  if (MASKED) {
    const int q_last = min(q0 + kQRows, N) - 1;
    const int w_last = min(qw + 32, N) - 1;
    int j_hi = nk;
    if (wl >= 0) {
      j_lo = max(0, q0 - wl) / kQCols;
      jw_lo = max(0, qw - wl) / kQCols;
      jf_lo = (max(0, w_last - wl) + kQCols - 1) / kQCols;
    }
    if (wr >= 0) {
      j_hi = min(nk, (q_last + wr) / kQCols + 1);
      jw_hi = (qw < N) ? min(nk, (w_last + wr) / kQCols + 1) : 0;
      jf_hi = min(jf_hi, qw + wr - (kQCols - 1) >= 0 ? (qw + wr - (kQCols - 1)) / kQCols + 1 : 0);
    }
    n_tiles = j_hi - j_lo;
  }
  // this row's visible keys [key_lo, key_hi]
  const int key_lo = (MASKED && wl >= 0) ? qrow - wl : 0;
  const int key_hi = (MASKED && wr >= 0) ? min(N - 1, qrow + wr) : N - 1;

  const LdsOffsets<D> off = lds_offsets<D>(lane);
  const unsigned lds0 = __builtin_amdgcn_readfirstlane(lds_offset_of(smem));
  // tile copies: kQCols / kRowsPerCopy instructions for K and as many for V;
  // instruction i is issued by wave i % 8
  auto copy_tile = [&](int j) __attribute__((always_inline)) {
    const int key0 = (j_lo + j) * kQCols;
    const int rows = min(kQCols, N - key0);
    const i32x4 rk = raw_rsrc(k + kv_head + (long long)key0 * kD, rows * kRowBytes);
    const i32x4 rv = raw_rsrc(v + kv_head + (long long)key0 * kD, rows * kRowBytes);
    const unsigned base = lds0 + (unsigned)((j % kQRing) * kQStage);
#pragma unroll
    for (int m = 0; m < kQCols / Gm::kRowsPerCopy / kQWaves; ++m) {
      const int i = wave + kQWaves * m;
      copy16_to_lds(rk, copy_voff<D>(lane, i), base + 1024 * i);
      copy16_to_lds(rv, copy_voff<D>(lane, i), base + kQTileBytes + 1024 * i);
    }
  };
  constexpr int kCopies = 2 * (kQCols / Gm::kRowsPerCopy / kQWaves);  // per wave per tile

  f32x16 dqacc[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  auto compute = [&](int j) __attribute__((always_inline)) {
    const int sbase = (j % kQRing) * kQStage;
    int krow[kKSteps], ktr[kDBlocks][2];
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) krow[s] = pin(off.row[s] + sbase);
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int u = 0; u < 2; ++u) ktr[db][u] = pin(off.tr[db][u] + sbase);
    const int ja = j_lo + j;  // key tile index
    const bool edge = ja < jf_lo || ja >= jf_hi;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T for keys 32*kb .. +31 of the tile,
      // [key x query]: the query is the lane; element i holds key
      // 64*j + 32*kb + 8*(i/4) + 4*half + (i%4).
      f32x16 sacc = {}, dpacc = {};
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) {
        const bf16x8 ka = *(const bf16x8*)(smem + krow[s] + 32 * kb * kRowBytes);
        sacc = mfma(ka, qf[s], sacc);
        const bf16x8 va = *(const bf16x8*)(smem + krow[s] + kQTileBytes + 32 * kb * kRowBytes);
        dpacc = mfma(va, gf[s], dpacc);
      }
      if (edge) {
        // a real branch: tiles inside every row's band skip the mask (the
        // empty volatile statement keeps the compiler from applying it to
        // every tile as selects)
        asm volatile("");
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = ja * kQCols + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          sacc[i] = (kk >= key_lo) & (kk <= key_hi) ? sacc[i] : -INFINITY;
        }
      }
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[i], c, nlse2));
        ds[i] = p * (dpacc[i] - dlt);
      }
      bf16x8 dsk[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int u = 0; u < 8; ++u) dsk[h][u] = (__bf16)ds[8 * h + u];
      // dQ^T += K^T dS^T: slot u of lane (query, half) in step h is key
      // 32*kb + 16*h + 8*(u/4) + 4*half + (u%4) in both operands.
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) {
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + ktr[db][0] + (32 * kb + 16 * h) * kRowBytes));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(smem + ktr[db][1] + (32 * kb + 16 * h + 8) * kRowBytes));
          dqacc[db] = mfma(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), dsk[h], dqacc[db]);
        }
    }
  };

  copy_tile(0);
  if (n_tiles > 1) copy_tile(1);
  for (int j = 0; j < n_tiles; ++j) {
    // tile j has landed (tile j+1 may still be in flight); after the
    // barrier every wave's copies of tile j are visible and every wave is
    // done with tile j-1, whose ring slot tile j+2 reuses
    wait_vmem(j + 1 < n_tiles ? kCopies : 0);
    __syncthreads();
    if (j + 2 < n_tiles) copy_tile(j + 2);
    if (j_lo + j >= jw_lo && j_lo + j < jw_hi) compute(j);
  }

  if (qrow >= N) return;
  const long long orow = head + (long long)qrow * kD;
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int dcol = 32 * db + 8 * a4 + 4 * half;
      const float x0 = dqacc[db][4 * a4] * scale, x1 = dqacc[db][4 * a4 + 1] * scale;
      const float x2 = dqacc[db][4 * a4 + 2] * scale, x3 = dqacc[db][4 * a4 + 3] * scale;
      if (GRAD_BF16) {
        const bf16x4 y = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
        *(u32x2*)((__bf16*)dq + orow + dcol) = __builtin_bit_cast(u32x2, y);
      } else {
        *(float4*)((float*)dq + orow + dcol) = make_float4(x0, x1, x2, x3);
      }
    }
}

template <int D, bool MASKED, bool GRAD_BF16>
hipError_t launch_bwd_t(const BwdArgs& a, float c) {
  const int BH = a.B * a.H;
  const int BHkv = a.B * a.Hkv;
  const int group = a.H / a.Hkv;
  const long long kv_grid = (long long)((a.N + kKVKeys - 1) / kKVKeys) * BHkv;
  const int T = (a.N + kQRows - 1) / kQRows;
  const long long q_grid = (long long)T * BH;
  if (kv_grid > 0x7fffffffLL || q_grid > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, MASKED, GRAD_BF16>), dim3((unsigned)kv_grid), dim3(kKVWaves * 64), 0, a.stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse,
                     a.delta, a.dk, a.dv, BHkv, a.N, c, a.scale, group, a.wl, a.wr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, MASKED, GRAD_BF16>), dim3((unsigned)q_grid), dim3(kQWaves * 64), 0, a.stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse,
                     a.delta, a.dq, BH, a.N, T, c, a.scale, group, a.wl, a.wr);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a) {
  const long long rows = (long long)a.B * a.H * a.N;
  constexpr int kRowsPerBlock = 256 / (D / 8);
  const long long dgrid = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (dgrid > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.o_bf16)
    hipLaunchKernelGGL((bwd_delta_kernel<D, true>), dim3((unsigned)dgrid), dim3(256), 0, a.stream, a.o,
                       (const __bf16*)a.dout, a.delta, rows);
  else
    hipLaunchKernelGGL((bwd_delta_kernel<D, false>), dim3((unsigned)dgrid), dim3(256), 0, a.stream, a.o,
                       (const __bf16*)a.dout, a.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const float c = fmaxf(a.scale * kLog2e, 1e-30f);
  if (a.wl >= 0 || a.wr >= 0)
    return a.grad_bf16 ? launch_bwd_t<D, true, true>(a, c) : launch_bwd_t<D, true, false>(a, c);
  return a.grad_bf16 ? launch_bwd_t<D, false, true>(a, c) : launch_bwd_t<D, false, false>(a, c);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a) {
  switch (a.d) {
    case 64: return launch_bwd_d<64>(a);
    case 128: return launch_bwd_d<128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa2
