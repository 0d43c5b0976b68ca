// FlashAttention-2 forward for bf16 inputs on gfx950 (MI355X): two kernels.
//
//  * fwd_kernel (plain, causal and sliding-window attention, also with
//    grouped key/value heads): 128-row query tiles on workgroups of four
//    wavefronts, two workgroups per compute unit, and ONE interleaved
//    MFMA/softmax instruction stream per wavefront and key tile.  Its own
//    comment block below gives the schedule.
//  * fwd_bf16_kernel (the split schedule's chunks, block-sparse lists, paged
//    decoding and the FP8 mode): 256-row query tiles on workgroups of eight
//    wavefronts in two groups that alternate matrix and vector phases.
//
// The products, layouts and online softmax described next are shared by
// both; the work decomposition and schedule paragraphs describe
// fwd_bf16_kernel.
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
// K/V tiles are copied from global memory straight into 3-deep (padded) LDS
// rings four phases before they are first read, and read by both groups.

#include "fa2_launch.h"

#include <atomic>
#include <cmath>
#include <cstdint>
#include <type_traits>

namespace fa2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWaves = kBf16Waves;      // 8: two groups of 4
constexpr int kGroupWaves = kWaves / 2;
constexpr int kRows = 32;               // query rows per wavefront
constexpr int kBr = kBf16BlockRows;     // query rows per workgroup
constexpr int kBc = kBf16BlockCols;     // keys per K/V tile
constexpr int kThreads = kWaves * 64;
constexpr int kRing = 3;                // K and V tiles resident per ring

template <int D, bool FP8K = false>
struct Geo {
  // LDS rows are padded so that every operand read is free of bank conflicts
  // and every per-lane address is one base register plus an immediate:
  //  * K (stride 2*D + 16 bytes): the 16 lanes of a b128 read phase read 16
  //    consecutive rows at the same column, which the 16-byte pad spreads
  //    over 16 distinct 16-byte slots of a 256-byte bank line;
  //  * V (stride 2*D, no pad): a half-wave transposing read touches 4
  //    consecutive rows x 64 bytes at one column; the 64-byte units of a row
  //    are stored XOR-permuted by a function of the row (vswz), which puts
  //    the 4 rows on 4 disjoint quarters of the bank line.  No pad means a
  //    V tile is D/8 copy instructions (64 lanes x 16 bytes) rather than
  //    D/8 + 4.
  //  (FP8 mode: K rows are D bytes of E4M3 codes, stride D + 16; the same
  //  16-slot argument holds for its 16-byte reads)
  static constexpr int kRowBytes = D * 2;
  static constexpr int kRowBytesK = FP8K ? D : D * 2;
  static constexpr int kStrideK = kRowBytesK + 16;
  static constexpr int kStrideV = kRowBytes;
  static constexpr int kTileK = kBc * kStrideK;
  static constexpr int kTileV = kBc * kStrideV;
  static constexpr int kLdsBytes = kRing * (kTileK + kTileV);
  static constexpr int kChunks = kRowBytes / 16;            // 16-byte data chunks per row
  static constexpr int kChunksK = kRowBytesK / 16;
  // A tile is copied by 64-lane instructions that each fill 64 consecutive
  // 16-byte LDS slots (pad slots included); instruction i goes to wave i % 8.
  static constexpr int kSlotsK = kStrideK / 16;              // 16-byte slots per K row
  static constexpr int kSlotsV = kStrideV / 16;
  static constexpr int kInstK = kBc * kSlotsK / 64;
  static constexpr int kInstV = kBc * kSlotsV / 64;
  static_assert(kBc * kSlotsK % 64 == 0 && kBc * kSlotsV % 64 == 0, "tiles must fill whole instructions");
  static constexpr int kKSteps = D / 16;                    // k-steps of the score MFMA
  static constexpr int kDBlocks = D / 32;                   // 32-row blocks of O^T
  // V row r keeps its 64-byte unit q (32 head dims) at unit q ^ vswz(r).
  // D = 128 (4 units, rows 256 bytes apart): rows r..r+3 need 4 distinct
  // units, vswz = r % 4.  D = 64 (2 units, 128-byte rows, two rows per
  // 256-byte bank line): rows r and r+2 share a half line, vswz = (r/2) % 2.
  static __device__ __forceinline__ int vswz(int r) { return D == 128 ? (r & 3) : ((r >> 1) & 1); }
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
// branches.  Both arguments must be wave-uniform; the size is passed through
// readfirstlane because clamps like max(0, min(a, b)) are selected as VALU
// instructions, and a descriptor in vector registers would turn every load
// into a loop over lanes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// cache policy of a buffer access: non-temporal (gfx950's nt bit)
constexpr int kCpolNT = 2;

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// Instruction-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kAhead = 4;  // LDS operand reads in flight ahead of the MFMAs

// sched_group_barrier takes constant arguments only; this maps a read count
// that is constant after unrolling onto one of them.
__device__ __forceinline__ void sched_ds_reads(int n) {
  if (n == 1) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
  else __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
}

// Schedule n_mfma MFMAs, each needing `reads` LDS reads, so that the reads
// run kAhead MFMAs ahead of their consumer.
template <int kNMfma, int kReads>
__device__ __forceinline__ void sched_reads_ahead() {
#pragma unroll
  for (int n = 0; n < kAhead; ++n) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kReads, 0);
#pragma unroll
  for (int n = 0; n < kNMfma; ++n) {
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    if (n + kAhead < kNMfma) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kReads, 0);
  }
}

// Copy 16 bytes per lane from global memory (wave-uniform 64-bit base in
// scalar registers plus a per-lane byte offset; no range check, callers
// clamp) straight into LDS: lane i's bytes land at LDS byte offset
// lds_offset + 16*i (lds_offset is wave-uniform).  global_load_lds lands
// from HBM markedly sooner than the buffer-descriptor form of the same copy
// (measured ~2,500 against ~3,900 cycles).  Written as inline assembly so
// that the compiler does not treat every later LDS read as dependent on the
// copy (it would wait for all outstanding copies); completion is tracked
// explicitly with wait_vmem and published with a workgroup barrier.
// Clobbers m0, which nothing else in these kernels uses.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(unsigned long long base, int voff, unsigned lds_offset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_offset), "v"(voff), "s"(base) : "memory", "m0");
}

// A wave-uniform 64-bit address in scalar registers.
__device__ __forceinline__ unsigned long long uniform_addr(const void* p) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(b & 0xffffffffu));
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  return ((unsigned long long)hi << 32) | lo;
}
#pragma clang diagnostic pop

// Byte offset of a __shared__ address within the workgroup's LDS.
__device__ __forceinline__ unsigned lds_offset_of(const void* p) {
  return (unsigned)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// s_waitcnt (gfx9 encoding): wait until at most n vector-memory operations
// of this wave are outstanding; LDS and export counters are left alone.
__device__ __forceinline__ void wait_vmem(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
    case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F76); break;
  }
}

// Pins a value to this point of the instruction stream.  asm volatile
// statements keep their order relative to the workgroup barriers, so this
// stops the compiler from moving the vector work of a phase (pure register
// arithmetic) across the barriers that delimit the phase.
template <typename T>
__device__ __forceinline__ T pin(T x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Lazy max correction: the reference max m of a row is only moved (and the
// banked l and O corrected) when the probabilities a tile gives against the
// current m sum to more than this in one half-row (32 keys), so every
// unnormalised probability stays in [0, 2^31], far inside fp32 range even
// summed over a million keys.  Any reference value gives the same softmax
// (the shift cancels between numerator and denominator); Saraf section 2.2:
// the correction is what keeps the answer exact.
constexpr float kTileSumLimit = 2147483648.0f;  // 2^31

template <int D, bool MASKED, bool OUT_BF16, bool SPARSE, bool PAGED, bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, void* __restrict__ o, float* __restrict__ lse,
                     int BH, int N, int T, float c, int poison, int group, int wl, int wr,
                     const SplitItem* __restrict__ items, float* __restrict__ part, int n_slots, int part_rows,
                     const int* __restrict__ sp_ptr, const unsigned* __restrict__ sp_ent, int n_layouts,
                     int n_entries, PagedArgs pg, const float* __restrict__ qsc,
                     const float* __restrict__ ksc) {
  using G = Geo<D, FP8>;
  // K tiles 0, 1 then V tiles 0, 1 (2-deep rings)
  __shared__ __attribute__((aligned(1024))) char smem[G::kLdsBytes];
  char* const lds_k = smem;
  char* const lds_v = smem + kRing * G::kTileK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform values are made explicit so they live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / kGroupWaves;  // 0 or 1 (group 1 runs one phase behind)
  const int gw = wave % kGroupWaves;   // position within the group = SIMD
  const int l32 = lane & 31;           // query column of this lane
  const int half = lane >> 5;          // which 4-key sub-rows of each 8-key group

  // Grid: workgroup -> (batch*head, query tile).  Causal tiles are issued
  // heaviest (latest rows) first.  With a split schedule (items != null)
  // the workgroup takes chunk blockIdx.x / BH of the schedule instead: a
  // query tile and a range of its key tiles, whose partial result goes to
  // partial slot `slot` (or straight to O and LSE when the tile is not
  // split).  Every field is clamped, so a malformed schedule cannot index
  // out of range.
  //
  // Paged decoding: BH counts (sequence, key/value head) groups; workgroup
  // (chunk c, group bh) takes the group's n_q newest tokens of its `group`
  // query heads (rows bh*nq_rows .. +nq_rows of q, o, lse: the heads of a
  // group are consecutive) against key tiles c*chunk_tiles .. +chunk_tiles
  // of the sequence's cache, and always writes a partial result (slot c).
  // Without a mask every query tile of a head does the same work; then,
  // when the heads come in multiples of 8, consecutive workgroups of one
  // XCD (blockIdx.x = x + 8r goes to XCD x) take the T tiles of one head
  // together, so the head's K and V are fetched into that XCD's L2 once
  // and read from there by its other tiles.
  const bool xcd_major = !MASKED && !SPARSE && !PAGED && items == nullptr && (BH & 7) == 0;
  const int xcd_r = (int)(blockIdx.x >> 3);
  const int bh = xcd_major ? (xcd_r / T) * 8 + (int)(blockIdx.x & 7) : (int)(blockIdx.x % BH);
  int t, ck_lo = 0, ck_hi = 1 << 30, slot = -1;
  int n_keys = N;         // keys this head attends over
  int nq_rows = N;        // query rows of this head (or group)
  int kvh = 0;            // paged: key/value head of the group
  const int* page_row = nullptr;
  if constexpr (PAGED) {
    const int b = bh / pg.kv_heads;
    kvh = bh % pg.kv_heads;
    n_keys = min(min(max(pg.ctx_lens[b], 0), pg.max_pages * pg.page_size), N);
    nq_rows = group * pg.n_q;
    page_row = pg.page_table + (long long)b * pg.max_pages;
    t = 0;
    slot = blockIdx.x / BH;
    ck_lo = slot * pg.chunk_tiles;
    ck_hi = ck_lo + pg.chunk_tiles;
    if (ck_lo * kBc >= n_keys) return;  // chunk past this sequence's context (uniform)
  } else if (items != nullptr) {
    const SplitItem it = items[blockIdx.x / BH];
    t = min(max(it.tile, 0), T - 1);
    ck_lo = max(it.kt_lo, 0);
    ck_hi = it.kt_hi;
    slot = it.slot < n_slots ? it.slot : -1;
  } else if (xcd_major) {
    t = xcd_r % T;
  } else {
    const int tr = blockIdx.x / BH;
    t = MASKED ? (T - 1 - tr) : tr;
  }

  const long long head = (long long)bh * nq_rows * D;
  // grouped key/value heads: `group` consecutive query heads share one
  // (paged: the cache base; the head is part of each tile's address)
  const long long kv_head = PAGED ? 0 : (long long)(bh / group) * N * D;
  // FP8: q and k hold E4M3 codes (one byte each) of the rotated Q and K with
  // one scale per (sequence, head); the MFMA sums code products, so the two
  // scales join the exp2 multiplier
  if constexpr (FP8) c = c * qsc[bh] * ksc[bh / group];
  const char* const kh = (const char*)k + kv_head * (FP8 ? 1 : 2);
  const char* const vh = (const char*)(v + kv_head);

  // Rows: the two wavefronts of a SIMD take adjacent 32-row slices, so the
  // causal work of the two groups stays balanced.
  const int q0 = t * kBr;
  const int qw = q0 + 64 * gw + 32 * grp;  // first row of this wavefront
  const int qrow = qw + l32;               // this lane's query row

  // Q rows of the wavefront as MFMA B operands (query = lane % 32,
  // head-dim slice 16*s + 8*half .. +7), held for the whole key loop.
  // Rows past N read as zeros.
  bf16x8 qf[G::kKSteps];
  i32x8 qf8[D / 64];  // FP8: query = lane % 32, codes of dims 64*s + 32*half .. +31
  if constexpr (FP8) {
    const int rows = max(0, min(kRows, nq_rows - qw));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)q + head + (long long)min(qw, nq_rows) * D, rows * D);
#pragma unroll
    for (int s = 0; s < D / 64; ++s) {
      const u32x4 lo = load16(rq, l32 * D + 64 * s + 32 * half);
      const u32x4 hi = load16(rq, l32 * D + 64 * s + 32 * half + 16);
      qf8[s] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  } else {
    const int rows = max(0, min(kRows, nq_rows - qw));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head + (long long)min(qw, nq_rows) * D, rows * D * 2);
#pragma unroll
    for (int s = 0; s < G::kKSteps; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, load16(rq, (l32 * D + 16 * s + 8 * half) * 2));
  }

  // Key tiles.  Key j is visible to query i iff i - wl <= j <= i + wr (a
  // negative bound: no limit on that side; causal is wl < 0, wr = 0).  The
  // workgroup streams key tiles j_lo .. j_lo + n_tiles - 1, those holding
  // any key visible to one of its rows; tiles above or below a wavefront's
  // rows are computed but fully masked.  This wavefront needs no mask on
  // tiles jf_lo .. jf_hi - 1, whose keys (all below N) every one of its rows
  // sees.
  const int nk = (n_keys + kBc - 1) / kBc;
  int j_lo = 0, n_tiles = nk, jf_lo = 0, jf_hi = n_keys / kBc;
  // paged: new token i of n_q sits at position n_keys - n_q + i and sees
  // the keys up to it; every row sees the tiles wholly below n_keys - n_q + 1
  if (PAGED) jf_hi = max(0, n_keys - pg.n_q + 1) / kBc;
  if (MASKED) {
    const int q_last = min(q0 + kBr, N) - 1;
    const int w_last = min(qw + kRows, N) - 1;
    if (wl >= 0) {
      j_lo = max(0, q0 - wl) / kBc;
      jf_lo = (max(0, w_last - wl) + kBc - 1) / kBc;
    }
    int j_hi = nk;
    if (wr >= 0) {
      j_hi = min(nk, (q_last + wr) / kBc + 1);
      jf_hi = min(jf_hi, qw + wr - (kBc - 1) >= 0 ? (qw + wr - (kBc - 1)) / kBc + 1 : 0);
    }
    n_tiles = j_hi - j_lo;
  }
  // Block-sparse: the key tiles come from the tile's list (entry = key tile
  // | wave-slice bits << 24; bit s set when the rows 32s .. 32s+31 of the
  // tile see keys of that tile), in the list's order.  Offsets and tile
  // indices are clamped into range.
  const int slice = 2 * gw + grp;  // this wavefront's 32-row slice of the tile
  int e0 = 0;
  if (SPARSE) {
    const long long pi = (long long)(bh % n_layouts) * T + t;
    e0 = min(max(sp_ptr[pi], 0), n_entries);
    const int e1 = min(max(sp_ptr[pi + 1], e0), n_entries);
    j_lo = 0;
    n_tiles = e1 - e0;
  }
  if (items != nullptr || PAGED) {
    // restrict the streamed key tiles to the chunk (at least one tile)
    const int j_hi = min(j_lo + n_tiles, max(ck_hi, ck_lo + 1));
    j_lo = min(max(j_lo, ck_lo), j_hi - 1);
    n_tiles = j_hi - j_lo;
  }
  // This row's visible keys, [key_lo, key_hi]: the mask is two compares per
  // score (no per-element branching on which bounds exist).
  const int key_lo = (MASKED && wl >= 0) ? qrow - wl : 0;
  const int key_hi = PAGED ? n_keys - pg.n_q + qrow % pg.n_q
                     : (MASKED && wr >= 0) ? min(N - 1, qrow + wr) : N - 1;
  // the key tile of step j, and whether this wavefront's rows see it
  auto tile_of = [&](int j) __attribute__((always_inline)) {
    if constexpr (SPARSE) return min((int)(sp_ent[e0 + j] & 0xFFFFFFu), nk - 1);
    else return j_lo + j;
  };
  auto wave_sees = [&](int j) __attribute__((always_inline)) {
    if constexpr (SPARSE) return ((sp_ent[e0 + j] >> (24 + slice)) & 1u) != 0u;
    else return true;
  };
  if (SPARSE && n_tiles == 0) {
    // no key tile: every row of the tile is empty (O = 0, LSE = -inf)
    if (qrow < N) {
      const long long orow = head + (long long)qrow * D;
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int dcol = 32 * db + 8 * a4 + 4 * half;
          if (OUT_BF16) *(u32x2*)((__bf16*)o + orow + dcol) = u32x2{0u, 0u};
          else *(float4*)((float*)o + orow + dcol) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      if (half == 0) lse[(long long)bh * N + qrow] = -INFINITY;
    }
    return;
  }

  // Tile copies: instruction i of a tile fills LDS slots [64i, 64i + 64);
  // slot u is (row u / slots-per-row, chunk u % slots-per-row); in K the
  // lanes that land on a row's pad slot fetch that row's chunk 0 (any
  // in-range address would do), in V each slot fetches the chunk the row's
  // unit permutation puts there.  Instruction i
  // is issued by wave i % 8; the per-lane source offsets do not depend on
  // the tile and are computed once.
  // bytes between consecutive keys in global memory (paged cache:
  // [page, slot, kv head, d], so H_kv rows of d apart)
  const int row_bytes = PAGED ? pg.kv_heads * G::kRowBytes : G::kRowBytes;
  const int row_bytes_k = PAGED ? row_bytes : G::kRowBytesK;
  constexpr int kCopyK = (G::kInstK + kWaves - 1) / kWaves;
  constexpr int kCopyV = (G::kInstV + kWaves - 1) / kWaves;
  int voff_k[kCopyK], voff_v[kCopyV];
#pragma unroll
  for (int k = 0; k < kCopyK; ++k) {
    const int u = (wave + k * kWaves) * 64 + lane;
    const int chunk = u % G::kSlotsK;
    voff_k[k] = (u / G::kSlotsK) * row_bytes_k + (chunk < G::kChunksK ? chunk : 0) * 16;
  }
#pragma unroll
  for (int k = 0; k < kCopyV; ++k) {
    // V slot u holds row u / kChunks, stored unit (u % kChunks) / 4, which is
    // the row's global unit (u % kChunks) / 4 ^ vswz(row)
    const int u = (wave + k * kWaves) * 64 + lane;
    const int row = u / G::kSlotsV, chunk = (u % G::kSlotsV) ^ (4 * G::vswz(row));
    voff_v[k] = row * row_bytes + chunk * 16;
  }
  const unsigned lds_k0 = __builtin_amdgcn_readfirstlane(lds_offset_of(lds_k)) + wave * 1024;
  const unsigned lds_v0 = __builtin_amdgcn_readfirstlane(lds_offset_of(lds_v)) + wave * 1024;
  auto copy_tile = [&](const char* src, int slot, int j, auto is_k) __attribute__((always_inline)) {
    constexpr bool K_TILE = decltype(is_k)::value;
    constexpr int kInst = K_TILE ? G::kInstK : G::kInstV;
    constexpr int kCopy = K_TILE ? kCopyK : kCopyV;
    const int key0 = tile_of(j) * kBc;
    const int rows = min(kBc, n_keys - key0);
    const int rb = K_TILE ? row_bytes_k : row_bytes;  // bytes between keys
    long long src_off = (long long)key0 * (K_TILE ? G::kRowBytesK : G::kRowBytes);
    if constexpr (PAGED) {
      // a tile lies in one page (page_size is a multiple of kBc)
      const int page = min(max(page_row[key0 / pg.page_size], 0), pg.n_pages - 1);
      src_off = (((long long)page * pg.page_size + key0 % pg.page_size) * pg.kv_heads * D + (long long)kvh * D) * 2;
    }
    const unsigned long long gsrc = uniform_addr(src + src_off);
    const unsigned base = (K_TILE ? lds_k0 + slot * G::kTileK : lds_v0 + slot * G::kTileV);
    if (poison) {
      // Debug: NaN over the 1 KiB blocks this wave's copies are about to
      // fill, completed before the copies are issued.  A read of the slot
      // before its copy lands, or a copy into a slot still being read,
      // then shows up as NaN in O.
      const u32x4 nan4 = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
#pragma unroll
      for (int k = 0; k < kCopy; ++k) {
        if (wave + k * kWaves < kInst)
          *(__attribute__((address_space(3))) u32x4*)(size_t)(base + k * kWaves * 1024 + 16 * lane) = nan4;
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the NaN is in LDS before any copy lands
    }
    // The last tile of a ragged sequence: rows past N are fetched from row
    // N-1 instead (global loads have no range check); those keys are masked
    // in the vector phase, so their K and V values never reach the output.
    const bool ragged = rows < kBc;
#pragma unroll
    for (int k = 0; k < kCopy; ++k) {
      if (wave + k * kWaves < kInst) {
        int vo = K_TILE ? voff_k[k] : voff_v[k];
        if (ragged) vo = min(vo / rb, rows - 1) * rb + vo % rb;
        copy16_to_lds(gsrc, vo, base + k * kWaves * 1024);
      }
    }
  };
  // copy instructions this wave issues per K (V) tile
  const int n_copy_k = (G::kInstK - wave + kWaves - 1) / kWaves;
  const int n_copy_v = (G::kInstV - wave + kWaves - 1) / kWaves;

  // Per-lane LDS offsets; everything else is an immediate.  K operand
  // (kb, s): row 32*kb + l32, columns 16*s + 8*half .. +7.  V transposing
  // read for (db, kb, h, u): lane i of each 16-lane group points at key row
  // (i / 4) of a 4-row slab and dcol 4*(i % 4) of a 16-column slab; lane i
  // then receives the 4 keys of one dcol (lane % 32).
  const int k_lane = l32 * G::kStrideK + 16 * half;
  // V: the lane's row within an 8-row slab is 4*half + (lane%16)/4; every
  // slab starts at a multiple of 8 rows, so vswz of the row is the lane's
  // own, and O^T block db (64-byte unit db) of the row sits at unit db ^ vswz.
  const int v_row = 4 * half + ((lane & 15) >> 2);
  const int v_col = (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  int v_lane[G::kDBlocks];
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db) v_lane[db] = v_row * G::kStrideV + v_col + 64 * (db ^ G::vswz(v_row));
  auto k_off = [&](int kb, int s) __attribute__((always_inline)) { return k_lane + 32 * kb * G::kStrideK + 32 * s; };
  // FP8 K operand (kb, s): row 32*kb + l32, codes of dims 64*s + 32*half .. +31
  const int k_lane8 = l32 * G::kStrideK + 32 * half;
  auto k_off8 = [&](int kb, int s) __attribute__((always_inline)) { return k_lane8 + 32 * kb * G::kStrideK + 64 * s; };
  auto read_k8 = [&](const char* kbuf, int kb, int s) __attribute__((always_inline)) {
    const u32x4 lo = *(const u32x4*)(kbuf + k_off8(kb, s));
    const u32x4 hi = *(const u32x4*)(kbuf + k_off8(kb, s) + 16);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E4M3 (format 0) and
  // unit block scales (E8M0 127 = 2^0)
  auto mfma_fp8 = [&](i32x8 a, i32x8 b, f32x16 acc) __attribute__((always_inline)) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
  };
  auto v_off = [&](int db, int kb, int h, int u) __attribute__((always_inline)) { return v_lane[db] + (32 * kb + 16 * h + 8 * u) * G::kStrideV; };

  f32x16 oacc[G::kDBlocks];
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  f32x16 sacc[2];
  bf16x8 pk[2][2];
  // Reference max of raw scores.  It is subtracted inside the score MFMA:
  // each chain starts from the accumulator negm = -m, so the vector phase
  // sees S - m and a probability is one multiply and one exp2.  m is set by
  // the first tile (0 until then).
  float m = 0.f;
  bool m_set = false;  // this row has met a visible key (m is its reference)
  f32x16 negm;
#pragma unroll
  for (int i = 0; i < 16; ++i) negm[i] = 0.f;
  float l = 0.f;     // running denominator over this lane's keys (fp32 P): for LSE
  float lb = 0.f;    // the same over the bf16-rounded P the second product uses: for O

  // ---- matrix phase of tile j: S_j = K_j Q^T, then O^T += V_{j-1}^T P_{j-1}^T
  // No branches here: for tiles past a wavefront's last row the scores are
  // computed but fully masked in the vector phase, so their P is 0.
  // Operands are read from LDS kAhead MFMAs ahead of their use.
  auto scores_mfma = [&](const char* kbuf) __attribute__((always_inline)) {
    if constexpr (FP8) {
#pragma unroll
      for (int n = 0; n < 2 * (D / 64); ++n)
        sacc[n & 1] = mfma_fp8(read_k8(kbuf, n & 1, n >> 1), qf8[n >> 1], n < 2 ? f32x16{} : sacc[n & 1]);
      return;
    }
    // MFMA n uses k-step s = n / 2 of block kb = n % 2 (two independent chains).
    constexpr int kN = 2 * G::kKSteps;
    auto read_k = [&](int n) __attribute__((always_inline)) { return *(const bf16x8*)(kbuf + k_off(n & 1, n >> 1)); };
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
  auto pv_mfma = [&](const char* vbuf) __attribute__((always_inline)) {
    // Key step (kb, h) covers keys 32*kb + 16*h + {0..15}; operand slot u
    // of lane (l32, half) is key 8*(u/4) + 4*half + (u%4) in both the P^T
    // operand (accumulator elements 8h..8h+7) and the V^T one.  MFMA n uses
    // key step n / kDBlocks on O^T block n % kDBlocks.
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
  // Tile j's K is in ring slot j % 3, tile j-1's V in slot (j - 1) % 3; the
  // slot is a compile-time constant in each third of the unrolled loops
  // below, so every LDS address is a base register plus an immediate.  The
  // 16 MFMAs of S_j and the 16 of O^T += V_{j-1}^T P_{j-1}^T form one stream
  // whose operand reads run kAhead MFMAs ahead across the boundary between
  // the two products, so the first O^T MFMA does not wait for a fresh read.
  // FP8: the stream is made of 16-byte operand units: 2 per score MFMA
  // (the halves of its 32-byte K operand), then one per O^T MFMA (as in the
  // bf16 stream); units are read kAhead ahead of their consumer.
  auto matrix_phase_fp8 = [&](auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    constexpr int kNS8 = 2 * (D / 64);    // score MFMAs (K = 64)
    constexpr int kNP = 4 * G::kDBlocks;  // MFMAs of O^T
    constexpr int kU = 2 * kNS8 + kNP;    // operand units
    const char* kbuf = lds_k + S * G::kTileK;
    const char* vbuf = lds_v + ((S + kRing - 1) % kRing) * G::kTileV;
    auto read_unit = [&](int u) __attribute__((always_inline)) {
      if (u < 2 * kNS8) {
        const int n = u >> 1;
        return *(const u32x4*)(kbuf + k_off8(n & 1, n >> 1) + 16 * (u & 1));
      }
      const int m = u - 2 * kNS8, db = m % G::kDBlocks, kb = (m / G::kDBlocks) >> 1, h = (m / G::kDBlocks) & 1;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbuf + v_off(db, kb, h, 0)));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbuf + v_off(db, kb, h, 1)));
      return __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    __builtin_amdgcn_s_setprio(1);
    u32x4 op[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) op[u] = read_unit(u);
    u32x4 first_half = {};
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const u32x4 a = op[u % kAhead];
      if (u + kAhead < kU) op[u % kAhead] = read_unit(u + kAhead);
      if (u < 2 * kNS8) {
        if ((u & 1) == 0) {
          first_half = a;
        } else {
          const int n = u >> 1;
          const i32x8 a8 = __builtin_bit_cast(i32x8, __builtin_shufflevector(first_half, a, 0, 1, 2, 3, 4, 5, 6, 7));
          sacc[n & 1] = mfma_fp8(a8, qf8[n >> 1], n < 2 ? negm : sacc[n & 1]);
        }
      } else {
        const int m = u - 2 * kNS8, db = m % G::kDBlocks, ks = m / G::kDBlocks;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pk[ks >> 1][ks & 1],
                                                          oacc[db], 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) sched_ds_reads(u < 2 * kNS8 ? 1 : 2);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (u >= 2 * kNS8 || (u & 1)) __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (u + kAhead < kU) sched_ds_reads(u + kAhead < 2 * kNS8 ? 1 : 2);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  auto matrix_phase = [&](auto slot) __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    if constexpr (FP8) {
      matrix_phase_fp8(slot);
      return;
    }
    constexpr int kNS = 2 * G::kKSteps;   // MFMAs of S_j
    constexpr int kNP = 4 * G::kDBlocks;  // MFMAs of O^T
    const char* kbuf = lds_k + S * G::kTileK;
    const char* vbuf = lds_v + ((S + kRing - 1) % kRing) * G::kTileV;
    // MFMA n < kNS: k-step n / 2 of score block n % 2 (two independent
    // chains).  MFMA kNS + m: key step m / kDBlocks (= (kb, h), keys
    // 32*kb + 16*h + {0..15}) on O^T block m % kDBlocks; operand slot u of
    // lane (l32, half) is key 8*(u/4) + 4*half + (u%4) in both the P^T
    // operand (accumulator elements 8h..8h+7) and the V^T one.
    auto read_op = [&](int n) __attribute__((always_inline)) {
      if (n < kNS) return *(const bf16x8*)(kbuf + k_off(n & 1, n >> 1));
      const int m = n - kNS, db = m % G::kDBlocks, kb = (m / G::kDBlocks) >> 1, h = (m / G::kDBlocks) & 1;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbuf + v_off(db, kb, h, 0)));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbuf + v_off(db, kb, h, 1)));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    __builtin_amdgcn_s_setprio(1);
    bf16x8 op[kAhead];
#pragma unroll
    for (int n = 0; n < kAhead; ++n) op[n] = read_op(n);
#pragma unroll
    for (int n = 0; n < kNS + kNP; ++n) {
      const bf16x8 a = op[n % kAhead];
      if (n + kAhead < kNS + kNP) op[n % kAhead] = read_op(n + kAhead);
      if (n < kNS) {
        sacc[n & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[n >> 1], n < 2 ? negm : sacc[n & 1], 0, 0, 0);
      } else {
        const int m = n - kNS, db = m % G::kDBlocks, ks = m / G::kDBlocks;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[ks >> 1][ks & 1], oacc[db], 0, 0, 0);
      }
    }
    // each MFMA is preceded by the reads of the MFMA kAhead later
#pragma unroll
    for (int n = 0; n < kAhead; ++n) sched_ds_reads(n < kNS ? 1 : 2);
#pragma unroll
    for (int n = 0; n < kNS + kNP; ++n) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (n + kAhead < kNS + kNP) sched_ds_reads(n + kAhead < kNS ? 1 : 2);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- vector phase of tile j: mask, P = exp2(...), row sums, correction ---
  // The scores arrive as S - m.  P = exp2((S - m)*c) is computed against the
  // current reference first; the tile's half-row sums then show whether m
  // must move (some sum above kTileSumLimit, or not finite), and only then
  // (or on the first tile, which sets m) is the row max formed, m moved, the
  // banked l and O^T corrected and P recomputed.
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  auto vector_phase = [&](int j) __attribute__((always_inline)) {
    const int ja = tile_of(j);  // key tile index
    const bool sees = wave_sees(j);
    if (!sees || ja < jf_lo || ja >= jf_hi) {
      // a real branch: tiles inside every row's band skip the mask (the
      // empty volatile statement keeps the compiler from applying it to
      // every tile as selects)
      asm volatile("");
      // element i of block kb holds key key0 + 32*kb + 8*(i/4) + 4*half + (i%4)
      const int key0 = ja * kBc;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          sacc[kb][i] = (key >= key_lo) & (key <= key_hi) & sees ? sacc[kb][i] : -INFINITY;
        }
    }
    sacc[0] = pin(sacc[0]);
    sacc[1] = pin(sacc[1]);
    // P = exp2((S - m)*c - sh*c), rounded to bf16 in pairs into the P^T
    // operand.  Two row sums: of the fp32 values (independent chains), which
    // LSE uses, and of the rounded bf16 pairs (v_dot2 with (1, 1)), which O
    // is divided by, so that the weights O is built from sum to one exactly.
    // (With the lazy max the largest P of a row is not exactly 1, so
    // dividing the rounded numerator by the unrounded sum would leave a
    // relative error of up to 2^-9 in O.)  Masked scores are -inf and c > 0,
    // so their probability is exactly 0.
    u32x4 w[2][2];
    float t, tb;
    // shift_c: subtract shc (= shift * c) in an FMA, or (common case) none
    auto probs = [&](auto shift_c, float shc) __attribute__((always_inline)) {
      constexpr bool kShift = decltype(shift_c)::value;
      float part[4] = {0.f, 0.f, 0.f, 0.f};
      float partb[2] = {0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(kShift ? fmaf(sacc[kb][i], c, -shc) : sacc[kb][i] * c);
          const float p1 = __builtin_amdgcn_exp2f(kShift ? fmaf(sacc[kb][i + 1], c, -shc) : sacc[kb][i + 1] * c);
          part[i & 3] += p0;
          part[(i & 3) + 1] += p1;
          const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
          partb[(i >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, partb[(i >> 1) & 1], false);
          w[kb][i >> 3][(i & 7) >> 1] = __builtin_bit_cast(unsigned, pp);
        }
      t = (part[0] + part[1]) + (part[2] + part[3]);
      tb = partb[0] + partb[1];
    };
    // Until some row of the wavefront has its reference (normally: the
    // wavefront's first key tile) every row takes the max path below, which
    // computes P itself; the pass against m = 0 would be thrown away.
    t = 0.f;
    if (__builtin_amdgcn_ballot_w64(m_set)) probs(std::false_type{}, 0.f);
    if (__builtin_amdgcn_ballot_w64(!m_set || !(t <= kTileSumLimit))) {
      // Row max of S - m in four independent chains (chain r takes the
      // elements e = 16*kb + i with e % 4 == r), then both halves of the row.
      auto el = [&](int e) __attribute__((always_inline)) { return sacc[e >> 4][e & 15]; };
      float mx[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) mx[r] = fmaxf(el(r), el(r + 4));
#pragma unroll
      for (int e = 8; e < 32; e += 8)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx[r] = fmaxf(fmaxf(mx[r], el(e + r)), el(e + r + 4));
      const float mt = max_halves(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
      // A row's first tile with a visible key sets m to that tile's row max
      // (l and O^T are still 0); later tiles move it up only.
      const bool has_key = mt > -INFINITY;
      const float sh = m_set ? fmaxf(mt, 0.f) : (has_key ? mt : 0.f);
      const float alpha = m_set ? __builtin_amdgcn_exp2f(-sh * c) : 0.f;
      m_set = m_set || has_key;
      m += sh;
#pragma unroll
      for (int i = 0; i < 16; ++i) negm[i] = -m;
      l *= alpha;
      lb *= alpha;
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      probs(std::true_type{}, sh * c);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      pk[kb][0] = pin(__builtin_bit_cast(bf16x8, w[kb][0]));
      pk[kb][1] = pin(__builtin_bit_cast(bf16x8, w[kb][1]));
    }
    lb = pin(lb + tb);
    l = pin(l + t);
  };

  using True_ = std::true_type;
  using False_ = std::false_type;
  // ---- prologue: K_0, K_1 and V_0 in LDS -----------------------------------
  copy_tile(kh, 0, 0, True_{});
  copy_tile(vh, 0, 0, False_{});
  if (n_tiles > 1) copy_tile(kh, 1, 1, True_{});
  wait_vmem(0);
  __syncthreads();

  // ---- phases ----------------------------------------------------------------
  // Phase p: group 0 runs the matrix phase of tile p/2 (p even) or the
  // vector phase of tile (p-1)/2 (p odd); group 1 does the same one phase
  // later.  K_j is read in phases 2j and 2j+1, V_j in phases 2j+2 and 2j+3.
  // From phase 2j on, the ring slots of K_{j-1} and V_{j-2} are dead, so
  // K_{j+2} and V_{j+1} are copied into them in step j (phase 2j for group
  // 1, phase 2j+1 for group 0: each group at the start of its vector phase);
  // both are first read in phase 2j+4.  Before the barrier that ends step j
  // each wave waits for its copies of step j-1, leaving those of step j in
  // flight.
  // Each group runs its own straight-line loop (unrolled by three for the
  // ring slot); both pass the same number of barriers.
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  auto issue = [&](int j, auto slot) __attribute__((always_inline)) {  // slot = j % 3
    constexpr int S = decltype(slot)::value;
    if (j + 2 < n_tiles) copy_tile(kh, (S + 2) % kRing, j + 2, True_{});
    if (j + 1 < n_tiles) copy_tile(vh, (S + 1) % kRing, j + 1, False_{});
  };
  // copies of step j (what may stay in flight at the end of step j)
  auto in_flight = [&](int j) __attribute__((always_inline)) {
    return (j + 2 < n_tiles ? n_copy_k : 0) + (j + 1 < n_tiles ? n_copy_v : 0);
  };
  // Tile 0 has no previous P*V: its matrix phase computes scores only.
  auto first_matrix_phase = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    scores_mfma(lds_k);
    sched_reads_ahead<2 * G::kKSteps, 1>();
    __builtin_amdgcn_s_setprio(0);
  };
  auto last_pv = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    switch ((n_tiles - 1) % kRing) {
      case 0: pv_mfma(lds_v); break;
      case 1: pv_mfma(lds_v + G::kTileV); break;
      default: pv_mfma(lds_v + 2 * G::kTileV); break;
    }
    __builtin_amdgcn_s_setprio(0);
  };
  if (grp == 0) {
    // Group 0 issues its copies of step j at the start of its vector phase
    // (phase 2j+1) rather than of its matrix phase: a copy stalls the wave
    // that issues it, and the vector phase has the slack.
    auto step = [&](int j, auto slot) __attribute__((always_inline)) {
      matrix_phase(slot);
      __syncthreads();
      issue(j, slot);
      vector_phase(j);
      wait_vmem(in_flight(j));
      __syncthreads();
    };
    first_matrix_phase();
    __syncthreads();
    issue(0, S0{});
    vector_phase(0);
    wait_vmem(in_flight(0));
    __syncthreads();
    int j = 1;
    for (; j + 2 < n_tiles; j += 3) {
      step(j, S1{});
      step(j + 1, S2{});
      step(j + 2, S0{});
    }
    if (j < n_tiles) step(j, S1{});
    if (j + 1 < n_tiles) step(j + 1, S2{});
    last_pv();
    __syncthreads();
    __syncthreads();
  } else {
    auto step = [&](int j, auto slot) __attribute__((always_inline)) {
      issue(j, slot);
      vector_phase(j - 1);
      __syncthreads();
      matrix_phase(slot);
      wait_vmem(in_flight(j));
      __syncthreads();
    };
    issue(0, S0{});
    __syncthreads();
    first_matrix_phase();
    wait_vmem(in_flight(0));
    __syncthreads();
    int j = 1;
    for (; j + 2 < n_tiles; j += 3) {
      step(j, S1{});
      step(j + 1, S2{});
      step(j + 2, S0{});
    }
    if (j < n_tiles) step(j, S1{});
    if (j + 1 < n_tiles) step(j + 1, S2{});
    vector_phase(n_tiles - 1);
    __syncthreads();
    last_pv();
    __syncthreads();
  }

  // ---- finalise: one division per row, then O and LSE ----------------------
  const float lt = sum_halves(l);
  const float ltb = sum_halves(lb);
  if (qrow >= nq_rows) return;
  if (slot >= 0) {
    // Partial result of a chunk: O normalised by the chunk's own rounded sum,
    // and the chunk's log-sums of the fp32 and of the rounded probabilities
    // (-inf, and O = 0, for a row that sees no key of the chunk); the merge
    // weighs the chunks by them (Mishra, "Another use of mergeable
    // statistics").
    const float inv = ltb > 0.f ? 1.0f / ltb : 0.f;
    float* const po = part + (((long long)bh * n_slots + slot) * part_rows + (qrow - q0)) * D;
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4)
        *(float4*)(po + 32 * db + 8 * a4 + 4 * half) =
            make_float4(oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv, oacc[db][4 * a4 + 2] * inv,
                        oacc[db][4 * a4 + 3] * inv);
    if (half == 0) {
      float2* const pl = (float2*)(part + (long long)BH * n_slots * part_rows * D) +
                         ((long long)bh * n_slots + slot) * part_rows + (qrow - q0);
      *pl = make_float2(lt > 0.f ? (m * c + log2f(lt)) * 0.69314718055994531f : -INFINITY,
                        ltb > 0.f ? (m * c + log2f(ltb)) * 0.69314718055994531f : -INFINITY);
    }
    return;
  }
  // (a row that saw no key -- possible only under a block-sparse mask --
  // has ltb = 0: O = 0 and LSE = -inf)
  const float inv = ltb > 0.f ? 1.0f / ltb : 0.f;
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
  if (half == 0) lse[(long long)bh * nq_rows + qrow] = (m * c + log2f(lt)) * 0.69314718055994531f;
}

// ---- the forward kernel (plain, causal and sliding-window masks) ------------
// Workgroups of 4 wavefronts (one per SIMD) own 128 query rows of one
// (batch, head), each wavefront 32 of them; two such workgroups share a
// compute unit, so the two wavefronts of a SIMD come from different
// workgroups and never wait for each other.
//
// Each wavefront runs ONE instruction stream per key tile j: the 16 MFMAs of
// O^T += V_{j-1}^T P_{j-1}^T, then the 16 of S_{j+1} = K_{j+1} Q^T, and after
// each MFMA a few VALU instructions of the softmax of S_j (the scores the
// previous tile's stream computed): the vector work of a tile runs in the
// shadow of the wavefront's own matrix work (Mishra, "FlashAttention-3:
// overlap work on Hopper": matrix operations interleaved with softmax work;
// "A pipeline is constrained by its slowest stage").  On gfx950 a wavefront
// that only issues MFMAs starves the VALU instructions of the other
// wavefront of its SIMD, so the overlap has to happen inside each stream.
//
// K and V tiles of 64 keys live in LDS rings of kR slots (slot = tile % kR;
// kR = 2 at d = 128, 3 at d = 64).  The stream of tile j copies K_{j+kR}
// and V_{j+kR-2} (global -> LDS, spread over its first MFMAs) into the
// slots of K_j and V_{j-2}, which nobody reads after the barrier that
// starts tile j; the barrier at the end of tile j, after each wavefront's
// wait for the copies the next stream reads, publishes them.
//
// A workgroup may own several (query tile, batch*head) items in turn
// (`sched`): 0 = one item, blockIdx.x; 1 = items g, g + G, g + 2G, ... (G
// workgroups) for grids of equal items larger than the chip holds at once,
// so that the cost of starting an item (its first loads, the store of its
// O) overlaps other work instead of hitting every compute unit at once
// (Saraf, section 2.3: keep every unit busy); 2 = a snake over the
// heaviest-first order (items g and 2G-1-g, then 2G+g, ...), which pairs
// long causal items with short ones into equal loads when there are at
// most two per workgroup slot.  The last P V product of an item reads no
// K, so its stream copies the next item's first kR K tiles into the K ring
// and loads the next item's Q rows: those loads are in flight while the
// item finishes and stores O, and the next item waits for them alone.
//
// O leaves through LDS (a quarter of the V ring per wavefront): each store
// instruction then writes whole rows of O instead of 32-byte pieces of 32
// rows, and exactly 1 KiB per instruction, so a wavefront issues a fixed
// number of stores per item.
constexpr int kW4 = kFwdWaves;          // wavefronts per workgroup (one per SIMD)
constexpr int kBr4 = kFwdBlockRows;     // query rows per workgroup
constexpr int kThreads4 = kW4 * 64;
constexpr int kAheadIL = 3;             // LDS operand reads in flight ahead of the MFMAs
static_assert(kBr4 == kW4 * kRows, "each wavefront owns 32 query rows");

// s_waitcnt with a compile-time vector-memory count of up to 63 (gfx9: the
// count's low 4 bits in bits 3:0, its high 2 bits in bits 15:14).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// K tiles of this kernel carry no pad inside their rows.  A copy
// instruction fills 1 KiB of LDS: here kRowsPerInst whole rows i, i + kSuper,
// i + 2 kSuper, ... of the tile (a "super-row"), followed by 16 unused bytes.
// Row r then sits at (r % kSuper) * 1040 + (r / kSuper) * row bytes: 16
// consecutive rows fall on 16 distinct 16-byte slots of a 256-byte bank
// line (the score MFMA's b128 operand reads are conflict-free), rows r and
// r + 32 are 512 bytes apart (a key block is an immediate offset), and a
// tile is exactly kSuper instructions, none of them spent on pad bytes.
template <int D, int R>
struct KRing {
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kRowsPerInst = 1024 / kRowBytes;  // 4 (d = 128), 8 (d = 64)
  static constexpr int kSuper = kBc / kRowsPerInst;      // copy instructions per tile
  static constexpr int kSuperBytes = 1024 + 16;
  static constexpr int kTile = kSuper * kSuperBytes;
  static constexpr int kBytes = (R * kTile + 1023) / 1024 * 1024;  // keeps the V ring 1 KiB aligned
  static constexpr int kBlock = (32 / kSuper) * kRowBytes;             // rows r -> r + 32
  static_assert(kSuper % kFwdWaves == 0 && 32 % kSuper == 0 && kBlock == 512, "K ring shape");
  static __device__ __forceinline__ int row_off(int r) { return (r % kSuper) * kSuperBytes + (r / kSuper) * kRowBytes; }
};

// Longest block-sparse list (key tiles of 64) the 128-row kernel takes: its
// compacted entries keep the key tile in 12 bits, and the list costs
// 2 bytes an entry of LDS (8 KiB, which two workgroups per CU still fit).
constexpr int kSparseMaxTiles = 4096;

template <int D, bool MASKED, bool OUT_BF16, bool PERSIST, bool SPARSE = false>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads4, kThreads4), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
               void* __restrict__ o, float* __restrict__ lse, int BH, int N, int T, float c, int poison, int group,
               int wl, int wr, int n_items, int sched, const int* __restrict__ sp_ptr,
               const unsigned* __restrict__ sp_ent, int n_layouts, int n_entries) {
  static_assert(!(SPARSE && PERSIST), "block-sparse items run one per workgroup");
  using G = Geo<D, false>;
  // Ring depth: at d = 128 two K and two V tiles (two workgroups per CU
  // fill 130 KiB of LDS), and stream j copies K_{j+2} and V_j, each needed
  // by stream j+1.  At d = 64 a stream is short, so a copy from HBM would
  // not land within one stream: three of each, and stream j copies
  // K_{j+3} and V_{j+1}, which have two streams to arrive.
  constexpr int kR = D == 64 ? 3 : 2;
  using KR = KRing<D, kR>;
  __shared__ __attribute__((aligned(1024))) char smem[KR::kBytes + kR * G::kTileV + (SPARSE ? 2 * kSparseMaxTiles : 0)];
  char* const lds_k = smem;
  char* const lds_v = smem + KR::kBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // Item -> (batch*head, query tile): causal and window tiles in heaviest
  // (latest rows) first order; without a mask and with heads in multiples of
  // 8, items x + 8r (whose workgroups all run on XCD x when the grid is a
  // multiple of 8) take the T tiles of one head, so its K and V are fetched
  // into that XCD's L2 once.
  const bool xcd_major = !MASKED && (BH & 7) == 0;
  const int n_wg = (int)gridDim.x, wg = (int)blockIdx.x;
  auto item_of = [&](int r) __attribute__((always_inline)) {
    const int i = (!PERSIST || sched == 0) ? (r == 0 ? wg : n_items)
                : sched == 1 ? wg + r * n_wg
                             : r * n_wg + ((r & 1) ? n_wg - 1 - wg : wg);
    return i < n_items ? i : -1;
  };
  const int n_keys = N;
  const int nk = (n_keys + kBc - 1) / kBc;
  // Key tiles j_lo .. j_lo + n_tiles - 1 hold a key some row of the
  // workgroup sees (key j visible to query i iff i - wl <= j <= i + wr, a
  // negative bound meaning no limit); this wavefront's rows see every key of
  // tiles jf_lo .. jf_hi - 1, which therefore need no mask.
  struct Item { int bh, t, j_lo, n_tiles, jf_lo, jf_hi; };
  auto geom = [&](int i) __attribute__((always_inline)) {
    Item it;
    it.bh = xcd_major ? ((i >> 3) / T) * 8 + (i & 7) : i % BH;
    it.t = xcd_major ? (i >> 3) % T : (MASKED ? (T - 1 - i / BH) : i / BH);
    const int q0 = it.t * kBr4, qw = q0 + 32 * wave;
    it.j_lo = 0;
    it.n_tiles = nk;
    it.jf_lo = 0;
    it.jf_hi = n_keys / kBc;
    if (MASKED) {
      const int q_last = min(q0 + kBr4, N) - 1;
      const int w_last = min(qw + kRows, N) - 1;
      if (wl >= 0) {
        it.j_lo = max(0, q0 - wl) / kBc;
        it.jf_lo = (max(0, w_last - wl) + kBc - 1) / kBc;
      }
      int j_hi = nk;
      if (wr >= 0) {
        j_hi = min(nk, (q_last + wr) / kBc + 1);
        it.jf_hi = min(it.jf_hi, qw + wr - (kBc - 1) >= 0 ? (qw + wr - (kBc - 1)) / kBc + 1 : 0);
      }
      it.n_tiles = j_hi - it.j_lo;
    }
    return it;
  };

  int item = item_of(0);
  if (item < 0) return;
  Item cur = geom(item);

  // Block-sparse: the item's key tiles are the entries of its 256-row
  // tile's list (entry = key tile | slice bits << 24, bit s set when the
  // rows 32s .. 32s+31 of the 256-row tile see that key tile) whose four
  // slice bits of this 128-row half are not all clear, in the list's order.
  // They are compacted once, 256 list entries per round of loads, into an
  // LDS array of 16-bit entries (key tile | the half's four slice bits << 12)
  // that every wavefront writes whole: the same values at the same places,
  // so each reads back its own writes without a barrier.  A lane register
  // holds a window of 128 of them, entry sp_base + i in bits 16*(i / 64) of
  // lane i % 64; lists longer than 128 move it on by 64 entries between
  // tile pairs (a pair looks at most 4 entries past its first tile).
  unsigned sp_list = 0u;
  int sp_base = 0;  // the list entry in bits 0..15 of lane 0 of sp_list
  int sp_bit = 0;   // this wavefront's slice bit in an entry
  unsigned short* const sp_lst = (unsigned short*)(smem + KR::kBytes + kR * G::kTileV);
  if constexpr (SPARSE) {
    const int T2 = (N + 255) / 256;
    const long long pi = (long long)(cur.bh % n_layouts) * T2 + cur.t / 2;
    const int e0 = min(max(sp_ptr[pi], 0), n_entries);
    const int ne = min(min(max(sp_ptr[pi + 1], e0), n_entries) - e0, kSparseMaxTiles);
    const int hbits = 24 + 4 * (cur.t & 1);
    int cnt = 0;
    for (int c0 = 0; c0 < ne; c0 += 256) {
      unsigned e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) e[u] = c0 + 64 * u + lane < ne ? sp_ent[e0 + c0 + 64 * u + lane] : 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool vis = ((e[u] >> hbits) & 0xFu) != 0u;
        const unsigned long long b = __builtin_amdgcn_ballot_w64(vis);
        const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(b >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)b, 0u));
        if (vis) sp_lst[pos] = (unsigned short)((e[u] & 0xFFFu) | (((e[u] >> hbits) & 0xFu) << 12));
        cnt += __builtin_popcountll(b);
      }
    }
    cur.n_tiles = cnt;
    sp_list = (unsigned)sp_lst[lane] | ((unsigned)sp_lst[64 + lane] << 16);
    sp_bit = 12 + wave;
    if (cur.n_tiles == 0) {
      // no key for any row of the item: O = 0, LSE = -inf
      constexpr int kEsz = OUT_BF16 ? 2 : 4;
      const int qw0 = cur.t * kBr4 + 32 * wave;
      const int rows = max(0, min(kRows, N - qw0));
      const long long hd = (long long)cur.bh * N * D;
      const __amdgpu_buffer_rsrc_t ro = make_rsrc((const char*)o + (hd + (long long)min(qw0, N) * D) * kEsz, rows * D * kEsz);
      const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int u = 0; u < kRows * D * kEsz / 1024; ++u)
        __builtin_amdgcn_raw_buffer_store_b128(z, ro, u * 1024 + 16 * lane, 0, 0);
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(lse + (long long)cur.bh * N + min(qw0, N), rows * 4);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(-INFINITY), rl, l32 * 4, 0, 0);
      return;
    }
  }
  // entry of the item's sparse tile jt (uniform, sp_base <= jt < sp_base + 128)
  auto sp_entry = [&](int jt) __attribute__((always_inline)) {
    const int i = jt - sp_base;
    return ((unsigned)__builtin_amdgcn_readlane((int)sp_list, i & 63) >> (16 * ((i >> 6) & 1))) & 0xFFFFu;
  };
  // before the tile pair starting at tile j: a list longer than the window
  // moves it on once j is 64 entries in
  auto sp_window = [&](int j) __attribute__((always_inline)) {
    if constexpr (SPARSE) {
      if (cur.n_tiles > sp_base + 128 && j >= sp_base + 64) {
        sp_base += 64;
        sp_list = (unsigned)sp_lst[min(sp_base + lane, kSparseMaxTiles - 1)] |
                  ((unsigned)sp_lst[min(sp_base + 64 + lane, kSparseMaxTiles - 1)] << 16);
      }
    }
  };
  // the current item's key tile of its tile jt (clamped to the last)
  auto key_tile = [&](int jt) __attribute__((always_inline)) {
    const int j = min(jt, cur.n_tiles - 1);
    if constexpr (SPARSE) return min((int)(sp_entry(j) & 0xFFFu), nk - 1);
    else return cur.j_lo + j;
  };
  // the current item's addresses and row bounds (set by enter())
  long long head = 0;
  const char* kh = nullptr;
  const char* vh = nullptr;
  int qw = 0, qrow = 0, key_lo = 0, key_hi = 0;
  auto enter = [&]() __attribute__((always_inline)) {
    head = (long long)cur.bh * N * D;
    const long long kv_head = (long long)(cur.bh / group) * N * D;
    kh = (const char*)(k + kv_head);
    vh = (const char*)(v + kv_head);
    qw = cur.t * kBr4 + 32 * wave;
    qrow = qw + l32;
    key_lo = (MASKED && wl >= 0) ? qrow - wl : 0;
    key_hi = (MASKED && wr >= 0) ? min(N - 1, qrow + wr) : N - 1;
  };

  // Q rows of the wavefront as MFMA B operands, held for an item's key loop;
  // rows past N read as zeros.
  bf16x8 qf[G::kKSteps];
  auto load_q = [&](long long head_, int qw_) __attribute__((always_inline)) {
    const int rows = max(0, min(kRows, N - qw_));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + head_ + (long long)min(qw_, N) * D, rows * D * 2);
#pragma unroll
    for (int s = 0; s < G::kKSteps; ++s) qf[s] = __builtin_bit_cast(bf16x8, load16(rq, (l32 * D + 16 * s + 8 * half) * 2));
  };

  // ---- copies: one instruction = 64 lanes x 16 bytes into 64 consecutive
  // 16-byte LDS slots; instruction i of a tile is issued by wavefront i % 4
  // (the layouts and per-lane source offsets are those of the other kernel)
  constexpr int kCopyK = KR::kSuper / kW4;
  constexpr int kCopyV = (G::kInstV + kW4 - 1) / kW4;
  constexpr int kMainK = KR::kSuper / kW4, kMainV = G::kInstV / kW4;
  constexpr int kRemK = 0, kRemV = G::kInstV % kW4;
  constexpr int kNC = kMainK + kMainV;  // copies spread through each tile's stream
  int voff_k[kCopyK], voff_v[kCopyV];
#pragma unroll
  for (int kk = 0; kk < kCopyK; ++kk) {
    // instruction wave + 4 kk: rows (wave + 4 kk) + kSuper * (lane / chunks)
    const int row = (wave + kk * kW4) + KR::kSuper * (lane / G::kChunks);
    voff_k[kk] = row * G::kRowBytes + (lane % G::kChunks) * 16;
  }
#pragma unroll
  for (int kk = 0; kk < kCopyV; ++kk) {
    const int u = (wave + kk * kW4) * 64 + lane;
    const int row = u / G::kSlotsV, chunk = (u % G::kSlotsV) ^ (4 * G::vswz(row));
    voff_v[kk] = row * G::kRowBytes + chunk * 16;
  }
  const unsigned lds_k0 = __builtin_amdgcn_readfirstlane(lds_offset_of(lds_k)) + wave * KR::kSuperBytes;
  const unsigned lds_v0 = __builtin_amdgcn_readfirstlane(lds_offset_of(lds_v)) + wave * 1024;
  // this wavefront's instruction kk of key tile jt (of the item whose keys
  // start at kbase, with tiles j_lo_ .. j_lo_ + n_tiles_ - 1) into ring slot
  // `slot`.  jt is clamped to the last tile (a copy past the end fetches it
  // again into a slot nobody reads); rows past N come from row N-1 and are
  // masked.
  // (Block-sparse: the current item's tiles only; its items are not
  // prefetched.)
  auto copy_k_of = [&](const char* kbase, int j_lo_, int n_tiles_, int jt, int slot, int kk) __attribute__((always_inline)) {
    const int key0 = (SPARSE ? key_tile(jt) : j_lo_ + min(jt, n_tiles_ - 1)) * kBc;
    const int rows = min(kBc, n_keys - key0);
    const unsigned long long gsrc = uniform_addr(kbase + (long long)key0 * G::kRowBytes);
    const int lim = __builtin_amdgcn_readfirstlane((rows - 1) * G::kRowBytes + G::kRowBytes - 16);
    copy16_to_lds(gsrc, min(voff_k[kk], lim), lds_k0 + slot * KR::kTile + kk * kW4 * KR::kSuperBytes);
  };
  auto copy_k = [&](int jt, int slot, int kk) __attribute__((always_inline)) {
    copy_k_of(kh, cur.j_lo, cur.n_tiles, jt, slot, kk);
  };
  auto copy_v = [&](int jt, int slot, int kk) __attribute__((always_inline)) {
    const int key0 = key_tile(jt) * kBc;
    const int rows = min(kBc, n_keys - key0);
    const unsigned long long gsrc = uniform_addr(vh + (long long)key0 * G::kRowBytes);
    const int lim = __builtin_amdgcn_readfirstlane((rows - 1) * G::kRowBytes + G::kRowBytes - 16);
    copy16_to_lds(gsrc, min(voff_v[kk], lim), lds_v0 + slot * G::kTileV + kk * kW4 * 1024);
  };
  // debug: NaN over this wave's destination blocks of the tile-j copies
  auto poison_slots = [&](int kslot, int vslot) __attribute__((always_inline)) {
    const u32x4 nan4 = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
#pragma unroll
    for (int kk = 0; kk < kCopyK; ++kk)
      *(__attribute__((address_space(3))) u32x4*)(size_t)(lds_k0 + kslot * KR::kTile + kk * kW4 * KR::kSuperBytes + 16 * lane) = nan4;
#pragma unroll
    for (int kk = 0; kk < kCopyV; ++kk)
      if (wave + kk * kW4 < G::kInstV)
        *(__attribute__((address_space(3))) u32x4*)(size_t)(lds_v0 + vslot * G::kTileV + kk * kW4 * 1024 + 16 * lane) = nan4;
    __builtin_amdgcn_s_waitcnt(0xC07F);
  };

  // ---- the next item (nxt, or -1), prefetched during the current item's
  // last P V product: its K tiles 0 .. kR-1 into K ring slots 0 .. kR-1, its Q
  // rows into qf.  Only its index stays live through the tile loop (its
  // geometry is recomputed where it is used): the looping kernel is short of
  // scalar registers.
  int nxt = -1;
  auto prefetch = [&]() __attribute__((always_inline)) {
    if (nxt >= 0) {
      const Item nx = geom(nxt);
      const char* const kbase = (const char*)(k + (long long)(nx.bh / group) * N * D);
#pragma unroll
      for (int kk = 0; kk < kCopyK; ++kk) {
        copy_k_of(kbase, nx.j_lo, nx.n_tiles, 0, 0, kk);
        copy_k_of(kbase, nx.j_lo, nx.n_tiles, 1, 1, kk);
        if (kR == 3) copy_k_of(kbase, nx.j_lo, nx.n_tiles, 2, 2, kk);
      }
      load_q((long long)nx.bh * N * D, nx.t * kBr4 + 32 * wave);
    }
  };

  // ---- LDS operand addresses: a per-lane base register plus an immediate
  // (ring slots are compile-time constants in the unrolled tile loop)
  const int k_lane = (int)lds_offset_of(lds_k) + KR::row_off(l32) + 16 * half;
  const int v_row = 4 * half + ((lane & 15) >> 2);
  const int v_col = (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  int v_lane[G::kDBlocks];
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
    v_lane[db] = (int)lds_offset_of(lds_v) + v_row * G::kStrideV + v_col + 64 * (db ^ G::vswz(v_row));

  f32x16 oacc[G::kDBlocks];
  f32x16 sA[2], sB[2];      // score tiles S_j (being turned into P) and S_{j+1} (being computed)
  u32x4 pk[2][2];           // P as bf16 pairs (P_j, produced by tile j's stream)
  float m = 0.f, mc = 0.f;  // reference max of the row (raw score units) and m*c
  bool m_set = false;
  float l = 0.f, lb = 0.f;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  constexpr int kNS = 2 * G::kKSteps;   // MFMAs of S
  constexpr int kNP = 4 * G::kDBlocks;  // MFMAs of O^T

  // One key tile's stream.  HAS_PV: O^T += V_{j-1}^T P_{j-1}^T;  HAS_S:
  // snext = K_{j+1} Q^T;  SOFT: P_j = exp2(S_j*c - m*c) from scur into pk,
  // with the row sums of the fp32 and of the bf16-rounded P;  copy_kv: bit 0
  // K_{j+kR}, bit 1 V_{j+kR-2}, bit 2 the next item's prefetch (at the first MFMA).
  // The sched_barrier after every MFMA and the empty asm statements that use
  // each softmax step's results keep the interleave the source order states
  // (the compiler would otherwise gather the VALU work).
  auto stream = [&](int j, auto slot, f32x16 (&scur)[2], f32x16 (&snext)[2],
                    auto has_pv, auto has_s, auto soft, auto copy_kv, float& tsum, float& tbsum) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;  // j % 2
    constexpr bool HAS_PV = decltype(has_pv)::value, HAS_S = decltype(has_s)::value;
    constexpr bool SOFT = decltype(soft)::value;
    constexpr bool COPY_K = decltype(copy_kv)::value & 1, COPY_V = (decltype(copy_kv)::value & 2) != 0;
    constexpr bool PREF = (decltype(copy_kv)::value & 4) != 0;
    constexpr int kNT = (HAS_PV ? kNP : 0) + (HAS_S ? kNS : 0);
    // ring slots: tile t sits in slot t % kR (a compile-time SL-derived
    // constant for kR = 2, uniform runtime values for kR = 3)
    int kKOff = (kR == 2 ? (SL + 1) % 2 : (j + 1) % 3) * KR::kTile;  // K_{j+1}
    int kVOff = (kR == 2 ? (SL + 1) % 2 : (j + 2) % 3) * G::kTileV;  // V_{j-1}
    if constexpr (kR != 2) {
      // whole offsets in scalar registers, so that each read base below
      // takes one add (the compiler would split the modulo over several)
      asm volatile("" : "+s"(kKOff));
      asm volatile("" : "+s"(kVOff));
    }
    const int kSlotW = kR == 2 ? SL : j % 3;                                // K_{j+kR}
    const int vSlotW = kR == 2 ? SL : (j + 1) % 3;                          // V_{j+kR-2}
    // per-lane read bases of this stream's slots, formed once (with runtime
    // slots the compiler would otherwise add the slot offset at every read)
    int k_base = k_lane + kKOff;
    int v_base[G::kDBlocks];
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db) v_base[db] = v_lane[db] + kVOff;
    if constexpr (kR != 2) {
      asm volatile("" : "+v"(k_base));
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db) asm volatile("" : "+v"(v_base[db]));
    }
    // A operand of stream MFMA n: for n < kNP (HAS_PV) V^T of key step
    // n / kDBlocks (keys 16*ks .. +15, transposing reads) for O^T block
    // n % kDBlocks; then K rows 32*(ns & 1) .. +31 at k-step ns / 2
    auto read_op = [&](int n) __attribute__((always_inline)) {
      if (HAS_PV && n < kNP) {
        const int db = n % G::kDBlocks, ks = n / G::kDBlocks, kb = ks >> 1, h = ks & 1;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)(v_base[db] + (32 * kb + 16 * h) * G::kStrideV));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(size_t)(v_base[db] + (32 * kb + 16 * h + 8) * G::kStrideV));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      const int ns = n - (HAS_PV ? kNP : 0);
      return *(const __attribute__((address_space(3))) bf16x8*)(size_t)(k_base + KR::kBlock * (ns & 1) + 32 * (ns >> 1));
    };
    // The softmax as a 3-stage pipeline over the 16 element pairs of a lane
    // (pair p: block p / 8, elements 2(p % 8) and +1).  Half-step 2u: exp2 of
    // pair u-1 and the exponent arguments of pair u; half-step 2u+1: sums
    // and bf16 packing of pair u-2.  36 half-steps, spread over all MFMAs
    // but the last four.
    float xs[2][2], es[2][2];  // [pair parity][element]
    float part[4] = {0.f, 0.f, 0.f, 0.f}, partb[2] = {0.f, 0.f};
    auto half_step = [&](int hs) __attribute__((always_inline)) {
      const int u = hs >> 1;
      if ((hs & 1) == 0) {
        if (u >= 1 && u <= 16) {
          const int pp_ = (u - 1) & 1;
          es[pp_][0] = __builtin_amdgcn_exp2f(xs[pp_][0]);
          es[pp_][1] = __builtin_amdgcn_exp2f(xs[pp_][1]);
          asm volatile("" :: "v"(es[pp_][0]), "v"(es[pp_][1]));  // keep the step at this point of the stream
        }
        if (u < 16) {
          xs[u & 1][0] = fmaf(scur[u >> 3][2 * (u & 7)], c, -mc);
          xs[u & 1][1] = fmaf(scur[u >> 3][2 * (u & 7) + 1], c, -mc);
          asm volatile("" :: "v"(xs[u & 1][0]), "v"(xs[u & 1][1]));
        }
      } else if (u >= 2) {
        const int p = u - 2, q_ = p & 1;
        const int i = 2 * (p & 7);
        part[i & 3] += es[q_][0];
        part[(i & 3) + 1] += es[q_][1];
        const bf16x2 pp = {(__bf16)es[q_][0], (__bf16)es[q_][1]};
        partb[(i >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, partb[(i >> 1) & 1], false);
        pk[p >> 3][i >> 3][(i & 7) >> 1] = __builtin_bit_cast(unsigned, pp);
        asm volatile("" :: "v"(part[i & 3]), "v"(part[(i & 3) + 1]), "v"(partb[(i >> 1) & 1]),
                     "v"(pk[p >> 3][i >> 3][(i & 7) >> 1]));
      }
    };
    constexpr int kHS = 36;
    // P_{j-1} as the O += V P MFMAs read it: the softmax overwrites pk with
    // P_j pair by pair while they run (where every write comes after the
    // last read of its element the two share registers)
    u32x4 pprev[2][2];
#pragma unroll
    for (int a0 = 0; a0 < 2; ++a0)
#pragma unroll
      for (int a1 = 0; a1 < 2; ++a1) pprev[a0][a1] = pk[a0][a1];
    bf16x8 op[kAheadIL];
    if constexpr (kNT > 0) {
#pragma unroll
      for (int n = 0; n < kAheadIL; ++n) op[n] = read_op(n);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < kNT; ++n) {
      const bf16x8 a = op[n % kAheadIL];
      if (n + kAheadIL < kNT) op[n % kAheadIL] = read_op(n + kAheadIL);
      if (HAS_PV && n < kNP) {
        const int db = n % G::kDBlocks, ks = n / G::kDBlocks;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, pprev[ks >> 1][ks & 1]), oacc[db], 0, 0, 0);
      } else {
        const int ns = n - (HAS_PV ? kNP : 0);
        snext[ns & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ns >> 1], ns < 2 ? f32x16{} : snext[ns & 1], 0, 0, 0);
      }
      if constexpr (SOFT) {
        // half-steps hs with floor(hs * kNTS / kHS) == n: spread over all
        // but the last four MFMAs, under which the last exponentials finish
        // before the tile's end reads their sums
        constexpr int kNTS = kNT > 8 ? kNT - 4 : kNT;
        if (n < kNTS) {
#pragma unroll
          for (int hs = (n * kHS + kNTS - 1) / kNTS; hs < ((n + 1) * kHS + kNTS - 1) / kNTS; ++hs) half_step(hs);
        }
      }
#pragma unroll
      for (int cc = 0; cc < kNC; ++cc)
        if (n == (kNT * cc) / (2 * kNC)) {
          if (cc < kMainK) {
            if constexpr (COPY_K) copy_k(j + kR, kSlotW, cc);
          } else {
            if constexpr (COPY_V) copy_v(j + kR - 2, vSlotW, cc - kMainK);
          }
        }
      if constexpr (PREF) {
        if (n == 0) prefetch();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (SOFT && kNT == 0) {
#pragma unroll
      for (int hs = 0; hs < kHS; ++hs) half_step(hs);
    }
    if constexpr (SOFT) {
      tsum = (part[0] + part[1]) + (part[2] + part[3]);
      tbsum = partb[0] + partb[1];
    }
  };

  // Mask of score tile j: only tiles this wavefront's rows do not all see
  // whole (window / causal edges, the ragged end of the sequence).  Element i
  // of block kb holds key 64*ja + 32*kb + 8*(i/4) + 4*half + (i%4).
  auto mask_tile = [&](int j, f32x16 (&sc)[2]) __attribute__((always_inline)) {
    const int ja = key_tile(j);
    if (SPARSE && !((sp_entry(j) >> sp_bit) & 1u)) {
      // block-sparse: this wavefront's rows see no key of the tile
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[kb][i] = -INFINITY;
    } else if (ja < cur.jf_lo || ja >= cur.jf_hi) {
      const int key0 = ja * kBc;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          sc[kb][i] = ((key >= key_lo) & (key <= key_hi)) ? sc[kb][i] : -INFINITY;
        }
    }
  };
  // End of tile j's softmax.  The reference max m of a row moves only when a
  // half-row's probabilities against it sum past kTileSumLimit (or on the
  // row's first visible tile): then m takes the row max, l and O^T (which
  // holds tiles < j) are multiplied by exp2((m_old - m_new)*c), and P_j is
  // recomputed -- the correction that keeps the result exact (Saraf, section
  // 2.2).
  auto settle = [&](f32x16 (&sc)[2], float tt, float tb) __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(!m_set || !(tt <= kTileSumLimit))) {
      auto el = [&](int e) __attribute__((always_inline)) { return sc[e >> 4][e & 15]; };
      float mx[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) mx[r] = fmaxf(el(r), el(r + 4));
#pragma unroll
      for (int e = 8; e < 32; e += 8)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx[r] = fmaxf(fmaxf(mx[r], el(e + r)), el(e + r + 4));
      const float mt = max_halves(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
      const bool has_key = mt > -INFINITY;
      const float nm = m_set ? fmaxf(m, mt) : (has_key ? mt : 0.f);
      const float alpha = m_set ? __builtin_amdgcn_exp2f((m - nm) * c) : 0.f;
      m_set = m_set || has_key;
      m = nm;
      mc = m * c;
      l *= alpha;
      lb *= alpha;
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      float part[4] = {0.f, 0.f, 0.f, 0.f}, partb[2] = {0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[kb][i], c, -mc));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[kb][i + 1], c, -mc));
          part[i & 3] += p0;
          part[(i & 3) + 1] += p1;
          const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
          partb[(i >> 1) & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, partb[(i >> 1) & 1], false);
          pk[kb][i >> 3][(i & 7) >> 1] = __builtin_bit_cast(unsigned, pp);
        }
      tt = (part[0] + part[1]) + (part[2] + part[3]);
      tb = partb[0] + partb[1];
    }
    l += tt;
    lb += tb;
  };

  using T_ = std::true_type;
  using F_ = std::false_type;
  using C0 = std::integral_constant<int, 0>;   // no copies
  using CV = std::integral_constant<int, 2>;   // V copies only
  using CKV = std::integral_constant<int, 3>;  // K and V copies
  using CP = std::integral_constant<int, 4>;   // the next item's prefetch
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // all of this wavefront's copy instructions of K (V) tile jt
  auto copy_k_all = [&](int jt, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < kCopyK; ++kk)
      copy_k(jt, slot, kk);
  };
  auto copy_v_all = [&](int jt, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < kCopyV; ++kk)
      if (wave + kk * kW4 < G::kInstV) copy_v(jt, slot, kk);
  };

  // Key tile j (SL = j % 2: S_j in sA for even j, sB for odd; ring slots
  // j % kR).
  auto tile = [&](int j, auto slot, auto has_pv, auto has_s, auto cp) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    constexpr bool COPY_K = decltype(cp)::value & 1, COPY_V = (decltype(cp)::value & 2) != 0;
    f32x16 (&scur)[2] = SL ? sB : sA;
    f32x16 (&snext)[2] = SL ? sA : sB;
    const int kSlotW = kR == 2 ? SL : j % 3, vSlotW = kR == 2 ? SL : (j + 1) % 3;
    if (poison) poison_slots(kSlotW, vSlotW);
    if (COPY_K && kRemK > 0 && wave < kRemK) copy_k(j + kR, kSlotW, kMainK);
    if (COPY_V && kRemV > 0 && wave < kRemV) copy_v(j + kR - 2, vSlotW, kMainV);
    mask_tile(j, scur);  // diagonal / window edges, and the ragged last tile
    float tt, tb;
    stream(j, slot, scur, snext, has_pv, has_s, T_{}, cp, tt, tb);
    settle(scur, tt, tb);
    if constexpr (kR == 2) {
      wait_vmem(0);
    } else {
      // this stream's copies may stay in flight (next needed two streams
      // on); the previous stream's, which the next one reads, must be in
      wait_vmem_n<(COPY_K ? kMainK : 0) + (COPY_V ? kMainV : 0)>();
    }
    __syncthreads();  // B_{j+1}
  };

  // Stores of one item: exactly kStores vector-memory instructions per
  // wavefront (rows past N are dropped by the buffer range, not by a
  // branch), so that the next item can wait for its prefetch alone.
  constexpr int kStores = (kRows * D * (OUT_BF16 ? 2 : 4)) / 1024 + 1;  // 1 KiB of O per instruction, then LSE
  // Issue priority falls with the workgroup's progress through its items:
  // two workgroups share each CU, and the older one wins issue arbitration
  // between equal priorities, so without this it runs ahead and the other
  // finishes its items alone on a half-empty CU (measured: 10-15 us apart in
  // a 59 us run of [32, 16, 512, 64] at d = 64).  A workgroup that falls a quarter of its items
  // behind now takes precedence until it catches up.
  const int n_rounds = !PERSIST ? 1 : sched == 1 ? (n_items - wg + n_wg - 1) / n_wg : (item_of(1) >= 0 ? 2 : 1);
  bool prefetched = false;
  // One item (the r-th of this workgroup); LAST: no item follows, so no
  // prefetch.
  auto item_body = [&](int r, auto last) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last)::value;
    if (PERSIST) {
      switch (min(3, 4 * r / n_rounds)) {
        case 0: __builtin_amdgcn_s_setprio(3); break;
        case 1: __builtin_amdgcn_s_setprio(2); break;
        case 2: __builtin_amdgcn_s_setprio(1); break;
        default: __builtin_amdgcn_s_setprio(0); break;
      }
    }
    enter();
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
    m = 0.f;
    mc = 0.f;
    m_set = false;
    l = 0.f;
    lb = 0.f;
    // ---- prologue: K_0 .. K_{kR-1} (and, for kR = 3, V_0) in LDS, S_0 computed
    if (!prefetched) {
      load_q(head, qw);
      copy_k_all(0, 0);
      copy_k_all(1, 1);
      if (kR == 3) copy_k_all(2, 2);
      wait_vmem(0);
    } else {
      wait_vmem_n<kStores>();  // the prefetch, not the previous item's stores
    }
    __syncthreads();
    // kR = 3: V_0 (needed two streams on), issued after the barrier since the
    // previous item staged its O in this part of the V ring
    if (kR == 3) copy_v_all(0, 0);
    {
      float d0, d1;
      stream(-1, S1{}, sB, sA, F_{}, T_{}, F_{}, C0{}, d0, d1);  // "tile -1": S_0 (slot 0) into sA
    }
    __syncthreads();  // B_0: nobody reads K_0 any more

    if (PERSIST) nxt = LAST ? -1 : item_of(r + 1);
    // Tiles past tile 0 go in pairs (ring slots 1, 0); a lone last tile
    // computes no S and copies no K.  (When the last tile ends a pair it
    // computes an unused S and its K copy fetches the last tile again.)
    tile(0, S0{}, F_{}, T_{}, CKV{});
    int j = 1;
    for (; j + 1 < cur.n_tiles; j += 2) {
      sp_window(j);
      tile(j, S1{}, T_{}, T_{}, CKV{});
      tile(j + 1, S0{}, T_{}, T_{}, CKV{});
    }
    if (j < cur.n_tiles) {
      // (kR = 3: the V tile this one would copy lies past the last)
      using CL = std::conditional_t<kR == 2, CV, C0>;
      tile(j, S1{}, T_{}, F_{}, CL{});
    }
    // the last O += V P: P_{n-1} with V_{n-1} (a stream "at tile n")
    {
      float d0, d1;
      using CF = std::conditional_t<PERSIST && !LAST, CP, C0>;
      if (cur.n_tiles & 1) stream(cur.n_tiles, S1{}, sA, sB, T_{}, F_{}, F_{}, CF{}, d0, d1);
      else stream(cur.n_tiles, S0{}, sA, sB, T_{}, F_{}, F_{}, CF{}, d0, d1);
    }

    // ---- finalise: one division per row (by the sum of the rounded P the
    // products used), then O and LSE = ln2 * (m*c + log2 l)
    const float lt = sum_halves(l);
    const float ltb = sum_halves(lb);
    const float inv = ltb > 0.f ? 1.0f / ltb : 0.f;
    const int rows = max(0, min(kRows, N - qw));
    constexpr int kEsz = OUT_BF16 ? 2 : 4;
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc((const char*)o + (head + (long long)min(qw, N) * D) * kEsz, rows * D * kEsz);
    // O goes out through LDS: the accumulator layout gives a lane 16-byte
    // pieces of one row, so a direct store instruction would write 32-byte
    // pieces of 32 rows; staged, each store instruction writes whole rows.
    // The stage is this wave's quarter of the V ring (free once every wave is
    // past its last P V product: the barrier below); rows of kStageCols
    // columns, their 16-byte units XOR-permuted by the row so that the
    // column-wise writes of the 32 rows spread over the banks.
    constexpr int kStageBytes = 2 * G::kTileV / kW4;               // per wave (V slots 0 and 1)
    constexpr int kStageCols = kStageBytes / (kRows * kEsz);        // columns per pass
    constexpr int kPasses = D / kStageCols;
    constexpr int kUnits = kStageCols * kEsz / 16;                  // 16-byte units per staged row
    constexpr int kRowsPerRead = 64 / kUnits;                       // rows per 64-lane read
    static_assert(kStageCols % 32 == 0 && D % kStageCols == 0 && kUnits <= 64 && 64 % kUnits == 0, "stage shape");
    char* const stage = lds_v + wave * kStageBytes;
    if constexpr (kR == 3) {
      // A last tile that ends a pair (an odd tile count) copied the last V
      // tile again into V slot n_tiles % 3, which may be part of the stage,
      // and the tile-end wait left that copy in flight: it must land before
      // the stage is written.  Only the next item's K and Q loads, issued
      // after it, may stay in flight.
      if (PERSIST && !LAST && nxt >= 0) wait_vmem_n<kR * kCopyK>();
      else wait_vmem_n<0>();
    }
    __syncthreads();  // every wave's last P V product has read the V ring
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
#pragma unroll
      for (int dbl = 0; dbl < kStageCols / 32; ++dbl) {
        const int db = ps * (kStageCols / 32) + dbl;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int col = 32 * dbl + 8 * a4 + 4 * half;  // first of this lane's 4 columns within the pass
          const int unit = (col * kEsz / 16) ^ (l32 % kUnits);
          char* const dst = stage + l32 * (kStageCols * kEsz) + unit * 16 + (col * kEsz) % 16;
          const float x0 = oacc[db][4 * a4 + 0] * inv, x1 = oacc[db][4 * a4 + 1] * inv;
          const float x2 = oacc[db][4 * a4 + 2] * inv, x3 = oacc[db][4 * a4 + 3] * inv;
          if (OUT_BF16) {
            const bf16x4 y = {(__bf16)x0, (__bf16)x1, (__bf16)x2, (__bf16)x3};
            *(__attribute__((address_space(3))) u32x2*)(size_t)lds_offset_of(dst) = __builtin_bit_cast(u32x2, y);
          } else {
            const u32x4 y = {__float_as_uint(x0), __float_as_uint(x1), __float_as_uint(x2), __float_as_uint(x3)};
            *(__attribute__((address_space(3))) u32x4*)(size_t)lds_offset_of(dst) = y;
          }
        }
      }
#pragma unroll
      for (int rd = 0; rd < kRows / kRowsPerRead; ++rd) {
        const int row = rd * kRowsPerRead + lane / kUnits, unit = lane % kUnits;
        const u32x4 y = *(const __attribute__((address_space(3))) u32x4*)(size_t)lds_offset_of(
            stage + row * (kStageCols * kEsz) + (unit ^ (row % kUnits)) * 16);
        // non-temporal: O is not read again here, and streaming it past the
        // caches leaves them to the K and V tiles other workgroups still read
        __builtin_amdgcn_raw_buffer_store_b128(y, ro, row * (D * kEsz) + ps * (kStageCols * kEsz) + unit * 16, 0, kCpolNT);
      }
    }
    // both halves of a row hold the same LSE; both store it
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(lse + (long long)cur.bh * N + min(qw, N), rows * 4);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint((m * c + log2f(lt)) * 0.69314718055994531f), rl, l32 * 4,
                                          0, 0);
  };
  if constexpr (PERSIST && D == 128) {
    // At most two items per workgroup here (schedule 2, heaviest with
    // lightest): the item body is inlined twice instead of looping, which
    // leaves the register allocator no state to carry round a loop.
    item_body(0, F_{});
    if (nxt >= 0) {
      prefetched = true;
      cur = geom(nxt);
      item_body(1, T_{});
    }
  } else {
    for (int r = 0;; ++r) {
      item_body(r, F_{});
      if (!PERSIST || nxt < 0) break;
      prefetched = true;
      cur = geom(nxt);
    }
  }
}

// Compute units of the current device (looked up once per device).
hipError_t compute_units(int* units) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> by_device[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int n = by_device[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (n <= 0) return hipErrorInvalidValue;
    by_device[dev].store(n, std::memory_order_relaxed);
  }
  *units = n;
  return hipSuccess;
}

template <int D, bool MASKED, bool OUT_BF16, bool SPARSE, bool PAGED = false, bool FP8 = false>
hipError_t launch_t(const FwdArgs& a) {
  const int T = (a.N + kBr - 1) / kBr;
  const long long grid = (long long)(a.items ? a.n_items : T) * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  // c = scale * log2(e), kept >= 1e-30 so that masked (-inf) scores give
  // exactly 0 even for scale == 0; any c that small already makes every
  // probability exactly 1 in fp32.
  const float c = fmaxf(a.scale * 1.4426950408889634f, 1e-30f);
  if constexpr (!SPARSE && !PAGED && !FP8) {
    if (a.items == nullptr) {
      // plain, causal and sliding-window forward: the 128-row kernel
      const int T4 = (a.N + kBr4 - 1) / kBr4;
      const long long items = (long long)T4 * a.B * a.H;
      if (items > 0x7fffffffLL) return hipErrorInvalidValue;
      int units = 0;
      const hipError_t eu = compute_units(&units);
      if (eu != hipSuccess) return eu;
      const FwdSchedule sc = fwd_schedule(items, units, MASKED && a.wl < 0, D);
      // the d = 128 looping kernel runs at most two items per workgroup
      if (D != 64 && (sc.sched == 1 || (sc.sched == 2 && 2 * sc.workgroups < items))) return hipErrorInvalidValue;
      auto kern = sc.sched == 0 ? fwd_kernel<D, MASKED, OUT_BF16, false> : fwd_kernel<D, MASKED, OUT_BF16, true>;
      hipLaunchKernelGGL(kern, dim3((unsigned)sc.workgroups), dim3(kThreads4), 0, a.stream, (const __bf16*)a.q,
                         (const __bf16*)a.k, (const __bf16*)a.v, a.o, a.lse, a.B * a.H, a.N, T4, c, a.poison ? 1 : 0,
                         a.H / a.Hkv, a.wl, a.wr, (int)items, sc.sched, (const int*)nullptr,
                         (const unsigned*)nullptr, 1, 0);
      return hipGetLastError();
    }
  }
  if constexpr (SPARSE && !PAGED && !FP8) {
    if (a.items == nullptr && a.N <= 64 * kSparseMaxTiles) {
      // block-sparse with at most kSparseMaxTiles key tiles per list: the
      // 128-row kernel, one item per workgroup (an item streams only the key
      // tiles its own rows see)
      const int T4 = (a.N + kBr4 - 1) / kBr4;
      const long long items = (long long)T4 * a.B * a.H;
      if (items > 0x7fffffffLL) return hipErrorInvalidValue;
      hipLaunchKernelGGL((fwd_kernel<D, MASKED, OUT_BF16, false, true>), dim3((unsigned)items), dim3(kThreads4), 0,
                         a.stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o, a.lse,
                         a.B * a.H, a.N, T4, c, a.poison ? 1 : 0, a.H / a.Hkv, a.wl, a.wr, (int)items, 0, a.sp_ptr,
                         a.sp_ent, a.n_layouts, a.n_entries);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, MASKED, OUT_BF16, SPARSE, PAGED, FP8>), dim3((unsigned)grid), dim3(kThreads), 0,
                     a.stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o, a.lse,
                     a.B * a.H, a.N, T, c, a.poison ? 1 : 0, a.H / a.Hkv, a.wl, a.wr,
                     (const SplitItem*)a.items, (float*)a.part, a.n_slots, kBr, a.sp_ptr, a.sp_ent,
                     a.n_layouts, a.n_entries, PagedArgs{}, a.q_scale, a.k_scale);
  return hipGetLastError();
}

template <int D, bool SPARSE>
hipError_t launch_s(const FwdArgs& a) {
  if (a.wl >= 0 || a.wr >= 0)
    return a.o_bf16 ? launch_t<D, true, true, SPARSE>(a) : launch_t<D, true, false, SPARSE>(a);
  return a.o_bf16 ? launch_t<D, false, true, SPARSE>(a) : launch_t<D, false, false, SPARSE>(a);
}

template <int D>
hipError_t launch_d(const FwdArgs& a) {
  if (a.fp8) {
    if (a.wl >= 0 || a.wr >= 0)
      return a.o_bf16 ? launch_t<D, true, true, false, false, true>(a) : launch_t<D, true, false, false, false, true>(a);
    return a.o_bf16 ? launch_t<D, false, true, false, false, true>(a) : launch_t<D, false, false, false, false, true>(a);
  }
  return a.sp_ptr ? launch_s<D, true>(a) : launch_s<D, false>(a);
}


// ---- merge of a split schedule's partial results -----------------------------
// A query tile whose key range was cut into chunks has, per chunk a, a
// partial output O_a (normalised by the chunk's own sum of rounded
// probabilities) and two log-sums per row: lse_a over the fp32
// probabilities and lseb_a over the rounded ones.  Exactly as in one pass,
//   O   = sum_a exp(lseb_a - lseb) O_a,   lseb = log sum_a exp(lseb_a),
//   LSE = log sum_a exp(lse_a)
// (Mishra, "Another use of mergeable statistics": the (max, sum) pairs of
// disjoint key sets combine associatively).  Workgroup: (chunk item, batch
// * head, quarter of the tile's rows); only the first chunk of a split tile
// merges, the other items exit at once.  Each row is D/4 lanes of four
// columns, so a row's partials are read as whole coalesced rows.
constexpr int kMergeThreads = 256;
constexpr int kMergeRowsPerGroup = kBr / 4;

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kMergeThreads) void split_merge_kernel(const SplitItem* __restrict__ items,
                                                                  const float* __restrict__ part, void* __restrict__ o,
                                                                  float* __restrict__ lse, int BH, int N, int T,
                                                                  int n_slots) {
  constexpr int kLanesPerRow = D / 4;
  constexpr int kRowsPerPass = kMergeThreads / kLanesPerRow;
  const int quarter = blockIdx.x % 4;
  const int rest = blockIdx.x / 4;
  const int bh = rest % BH;
  const SplitItem it = items[rest / BH];
  if (it.slot < 0 || it.slot >= n_slots || it.slot != it.slot0) return;
  const int t = min(max(it.tile, 0), T - 1);
  const int s0 = it.slot0;
  const int np = min(it.n_parts, n_slots - s0);
  const int c4 = 4 * (threadIdx.x % kLanesPerRow);
  const float* const pbase = part + (long long)bh * n_slots * kBr * D;
  const float2* const lbase = (const float2*)(part + (long long)BH * n_slots * kBr * D) + (long long)bh * n_slots * kBr;
  for (int r = quarter * kMergeRowsPerGroup + threadIdx.x / kLanesPerRow; r < (quarter + 1) * kMergeRowsPerGroup;
       r += kRowsPerPass) {
    const int row = t * kBr + r;
    if (row >= N) break;
    float mb = -INFINITY, ml = -INFINITY;
    for (int a = 0; a < np; ++a) {
      const float2 x = lbase[(long long)(s0 + a) * kBr + r];
      ml = fmaxf(ml, x.x);
      mb = fmaxf(mb, x.y);
    }
    float sl = 0.f, sb = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int a = 0; a < np; ++a) {
      const float2 x = lbase[(long long)(s0 + a) * kBr + r];
      if (x.x > -INFINITY) sl += expf(x.x - ml);
      if (x.y > -INFINITY) {
        const float wgt = expf(x.y - mb);
        const float4 y = *(const float4*)(pbase + ((long long)(s0 + a) * kBr + r) * D + c4);
        sb += wgt;
        acc.x = fmaf(wgt, y.x, acc.x);
        acc.y = fmaf(wgt, y.y, acc.y);
        acc.z = fmaf(wgt, y.z, acc.z);
        acc.w = fmaf(wgt, y.w, acc.w);
      }
    }
    const float inv = sb > 0.f ? 1.0f / sb : 0.f;
    const long long orow = (long long)bh * N * D + (long long)row * D + c4;
    if (OUT_BF16) {
      bf16x4 y = {(__bf16)(acc.x * inv), (__bf16)(acc.y * inv), (__bf16)(acc.z * inv), (__bf16)(acc.w * inv)};
      *(u32x2*)((__bf16*)o + orow) = __builtin_bit_cast(u32x2, y);
    } else {
      *(float4*)((float*)o + orow) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (c4 == 0) lse[(long long)bh * N + row] = sl > 0.f ? ml + logf(sl) : -INFINITY;
  }
}

// Merge of paged decoding's chunks: one workgroup per (sequence, key/value
// head) group; the group's rows, its chunk count from the sequence's
// context length, the same combination as split_merge_kernel.  A row that
// saw no key in any chunk (or a sequence with no key) gets O = 0, LSE = -inf.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const float* __restrict__ part,
                                                                   void* __restrict__ o, float* __restrict__ lse,
                                                                   PagedArgs pg, int groups, int nq_rows,
                                                                   int n_slots, int max_keys) {
  constexpr int kLanesPerRow = D / 4;
  constexpr int kRowsPerPass = kMergeThreads / kLanesPerRow;
  const int bh = blockIdx.x;
  const int b = bh / pg.kv_heads;
  const int n_keys = min(min(max(pg.ctx_lens[b], 0), pg.max_pages * pg.page_size), max_keys);
  const int nk = (n_keys + kBc - 1) / kBc;
  const int np = min((nk + pg.chunk_tiles - 1) / pg.chunk_tiles, n_slots);
  const int c4 = 4 * (threadIdx.x % kLanesPerRow);
  const float* const pbase = part + (long long)bh * n_slots * nq_rows * D;
  const float2* const lbase = (const float2*)(part + (long long)groups * n_slots * nq_rows * D) +
                              (long long)bh * n_slots * nq_rows;
  for (int r = threadIdx.x / kLanesPerRow; r < nq_rows; r += kRowsPerPass) {
    float mb = -INFINITY, ml = -INFINITY;
    for (int a = 0; a < np; ++a) {
      const float2 x = lbase[(long long)a * nq_rows + r];
      ml = fmaxf(ml, x.x);
      mb = fmaxf(mb, x.y);
    }
    float sl = 0.f, sb = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int a = 0; a < np; ++a) {
      const float2 x = lbase[(long long)a * nq_rows + r];
      if (x.x > -INFINITY) sl += expf(x.x - ml);
      if (x.y > -INFINITY) {
        const float wgt = expf(x.y - mb);
        const float4 y = *(const float4*)(pbase + ((long long)a * nq_rows + r) * D + c4);
        sb += wgt;
        acc.x = fmaf(wgt, y.x, acc.x);
        acc.y = fmaf(wgt, y.y, acc.y);
        acc.z = fmaf(wgt, y.z, acc.z);
        acc.w = fmaf(wgt, y.w, acc.w);
      }
    }
    const float inv = sb > 0.f ? 1.0f / sb : 0.f;
    const long long orow = ((long long)bh * nq_rows + r) * D + c4;
    if (OUT_BF16) {
      bf16x4 y = {(__bf16)(acc.x * inv), (__bf16)(acc.y * inv), (__bf16)(acc.z * inv), (__bf16)(acc.w * inv)};
      *(u32x2*)((__bf16*)o + orow) = __builtin_bit_cast(u32x2, y);
    } else {
      *(float4*)((float*)o + orow) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (c4 == 0) lse[(long long)bh * nq_rows + r] = sl > 0.f ? ml + logf(sl) : -INFINITY;
  }
}

template <int D, bool OUT_BF16>
hipError_t launch_paged_t(const FwdArgs& a) {
  const int groups = a.B * a.Hkv;
  const int nq_rows = (a.H / a.Hkv) * a.paged.n_q;
  const long long grid = (long long)a.n_slots * groups;
  if (grid > 0x7fffffffLL || grid < 1) return hipErrorInvalidValue;
  const float c = fmaxf(a.scale * 1.4426950408889634f, 1e-30f);
  hipError_t e;
  if (nq_rows <= 128) {
    // up to four blocks of 32 rows: the lighter one-wavefront-per-chunk kernel
    e = launch_decode_waves(a);
  } else {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, false, false, false, true, false>), dim3((unsigned)grid), dim3(kThreads), 0,
                       a.stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, a.o, a.lse, groups, a.N,
                       1, c, a.poison ? 1 : 0, a.H / a.Hkv, -1, -1, (const SplitItem*)nullptr, (float*)a.part,
                       a.n_slots, nq_rows, (const int*)nullptr, (const unsigned*)nullptr, 1, 0, a.paged,
                       (const float*)nullptr, (const float*)nullptr);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D, OUT_BF16>), dim3((unsigned)groups), dim3(kMergeThreads), 0, a.stream,
                     (const float*)a.part, a.o, a.lse, a.paged, groups, nq_rows, a.n_slots, a.N);
  return hipGetLastError();
}

template <int D>
hipError_t launch_merge_d(const FwdArgs& a) {
  const int T = (a.N + kBr - 1) / kBr;
  const long long grid = 4LL * a.n_items * a.B * a.H;
  if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
  auto kern = a.o_bf16 ? split_merge_kernel<D, true> : split_merge_kernel<D, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kMergeThreads), 0, a.stream, (const SplitItem*)a.items,
                     (const float*)a.part, a.o, a.lse, a.B * a.H, a.N, T, a.n_slots);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  switch (a.d) {
    case 64: return launch_d<64>(a);
    case 128: return launch_d<128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_paged(const FwdArgs& a) {
  switch (a.d) {
    case 64: return a.o_bf16 ? launch_paged_t<64, true>(a) : launch_paged_t<64, false>(a);
    case 128: return a.o_bf16 ? launch_paged_t<128, true>(a) : launch_paged_t<128, false>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_split_merge(const FwdArgs& a) {
  if (a.items == nullptr || a.n_slots <= 0) return hipSuccess;
  switch (a.d) {
    case 64: return launch_merge_d<64>(a);
    case 128: return launch_merge_d<128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa2
