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
// (lane % 32) for 32 of the 64 keys: row reductions are in-lane plus one
// exchange between the two 32-lane halves (v_permlane32_swap).  The
// probabilities stay in registers in the layout the second product needs as
// its B operand:
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
// m is moved (and l and O^T multiplied by exp2((m_old - m_new)*c), the
// correction that keeps the result exact) only when the probabilities
// against the current m would grow past a bound; the division by l happens
// once, when the query tile is finished (Saraf section 2.2).  Causal key
// tiles entirely above a wavefront's rows are neither multiplied nor (when
// above the whole workgroup's rows) loaded; only the tile crossing the
// diagonal, or the ragged end of the sequence, is masked.
//
// Schedule (where gfx950 differs from the pages' A100 design): the vector
// work of the softmax costs about a third of the matrix work of a tile, and
// one wavefront alone issues vector instructions at only about half the
// SIMD's rate, so every wavefront runs a software pipeline that keeps both
// kinds of work in one instruction stream: while it computes the
// probabilities of tile j, its matrix core computes S of tile j+1 and
// O += V P of tile j-1, with three or four vector instructions issued
// between consecutive MFMAs.  The two wavefronts of a SIMD run the same
// pipeline and share its matrix core.  K/V tiles are copied from global
// memory straight into 3-deep (padded) LDS rings two iterations before
// they are read; one workgroup barrier per iteration publishes the copies
// and frees the ring slots.

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
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kWaves = kBf16Waves;      // 8, two per SIMD
constexpr int kRows = 32;               // query rows per wavefront
constexpr int kBr = kBf16BlockRows;     // query rows per workgroup
constexpr int kBc = kBf16BlockCols;     // keys per K/V tile
constexpr int kThreads = kWaves * 64;
constexpr int kRing = 3;                // K and V tiles resident per ring

template <int D>
struct Geo {
  // LDS rows are padded so that every operand read is free of bank conflicts
  // and every per-lane address is one base register plus an immediate:
  //  * K (stride 2*D + 16 bytes): the 16 lanes of a b128 read phase read 16
  //    consecutive rows at the same column, which the 16-byte pad spreads
  //    over 16 distinct 16-byte slots of a 256-byte bank line;
  //  * V (stride 2*D + 64 bytes): a half-wave transposing read touches 4
  //    rows x 64 bytes, which the 64-byte pad puts on 4 disjoint quarters.
  static constexpr int kRowBytes = D * 2;
  static constexpr int kStrideK = kRowBytes + 16;
  static constexpr int kStrideV = kRowBytes + 64;
  static constexpr int kTileK = kBc * kStrideK;
  static constexpr int kTileV = kBc * kStrideV;
  static constexpr int kLdsBytes = kRing * (kTileK + kTileV);
  static constexpr int kChunks = kRowBytes / 16;            // 16-byte data chunks per row
  // A tile is copied by 64-lane instructions that each fill 64 consecutive
  // 16-byte LDS slots (pad slots included); instruction i goes to wave i % 8.
  static constexpr int kSlotsK = kStrideK / 16;              // 16-byte slots per K row
  static constexpr int kSlotsV = kStrideV / 16;
  static constexpr int kInstK = kBc * kSlotsK / 64;
  static constexpr int kInstV = kBc * kSlotsV / 64;
  static_assert(kBc * kSlotsK % 64 == 0 && kBc * kSlotsV % 64 == 0, "tiles must fill whole instructions");
  static constexpr int kKSteps = D / 16;                    // k-steps of the score MFMA
  static constexpr int kDBlocks = D / 32;                   // 32-row blocks of O^T
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

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

constexpr int kAhead = 4;  // LDS operand reads in flight ahead of the MFMAs

// Raw buffer descriptor as four scalar registers, for the LDS copy below.
__device__ __forceinline__ i32x4 raw_rsrc(const void* base, int bytes) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(base);
  i32x4 r = {__builtin_amdgcn_readfirstlane((int)(b & 0xffffffffu)),
             __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xffffu)),
             __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
  return r;
}

// Copy 16 bytes per lane from global memory (buffer rsrc, byte offset
// voff; zeros past the end) straight into LDS: lane i's bytes land at LDS
// byte offset lds_offset + 16*i (lds_offset is wave-uniform).  Written as inline assembly so that the compiler does not
// treat every later LDS read as dependent on the copy (it would wait for all
// outstanding copies); completion is tracked explicitly with wait_vmem and
// published with a workgroup barrier.  Clobbers m0, which nothing else in
// these kernels uses.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(i32x4 rsrc, int voff, unsigned lds_offset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_offset), "v"(voff), "s"(rsrc) : "memory", "m0");
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

// Lazy max correction: the reference max m of a row is only moved (and the
// banked l and O corrected) when a tile's row max exceeds it by more than
// this many powers of two, so the unnormalised probabilities stay in
// [0, 2^32], far inside fp32 range even summed over a million keys.  Any
// reference value gives the same softmax (the shift cancels between
// numerator and denominator); Saraf section 2.2: the correction is what
// keeps the answer exact.
constexpr float kRescaleThreshold = 32.0f;

typedef const __attribute__((address_space(3))) char* lds_cptr;

// Hides x from the optimiser, so that a per-stage LDS base stays one
// register and every operand read of the stage is that register plus an
// immediate offset (rather than one register per read, hoisted out of the
// key loop).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Pins a value to this point of the instruction stream: the vector work of
// a pipeline stage must neither be hoisted above the barrier that starts
// the stage nor sunk below its MFMAs, or it would no longer interleave with
// them.  (asm volatile statements keep their order relative to barriers.)
template <typename T>
__device__ __forceinline__ T pin(T x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                     const __bf16* __restrict__ v, void* __restrict__ o, float* __restrict__ lse,
                     int BH, int N, int T, float c) {
  using G = Geo<D>;
  constexpr int kNPv = 4 * G::kDBlocks;  // MFMAs of O^T += V^T P^T per tile
  constexpr int kNS = 2 * G::kKSteps;    // MFMAs of S^T = K Q^T per tile
  // K ring (3 tiles) then V ring (3 tiles)
  __shared__ __attribute__((aligned(1024))) char smem[G::kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform values are made explicit so they live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  const int q0 = t * kBr;
  const int qw = q0 + kRows * wave;  // first row of this wavefront
  const int qrow = qw + l32;         // this lane's query row

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

  // Key tiles: the workgroup streams n_tiles of them; this wavefront
  // multiplies the first n_w (causal: those starting at or below its last
  // row) and masks those from n_full on.  Because a wavefront's 32 rows
  // start at a multiple of 32, n_full >= n_w - 1: only its last tile can
  // need the mask.
  const int nk = (N + kBc - 1) / kBc;
  int n_tiles = nk, n_w = (qw < N) ? nk : 0, n_full = N / kBc;
  if (CAUSAL) {
    n_tiles = min(nk, (min(q0 + kBr, N) - 1) / kBc + 1);
    n_w = (qw < N) ? min(nk, (min(qw + kRows, N) - 1) / kBc + 1) : 0;
    n_full = min(n_full, (qw + 1) / kBc);
  }
  const bool mask_last = n_full < n_w;

  // Tile copies: instruction i of a tile fills LDS slots [64i, 64i + 64);
  // slot u is (row u / slots-per-row, chunk u % slots-per-row), and the
  // lanes that land on a row's pad slots fetch that row's chunk 0 (any
  // in-range address would do).  Keys past N read as zeros.  Instruction i
  // is issued by wave i % 8; the per-lane source offsets do not depend on
  // the tile and are computed once.
  constexpr int kCopyK = (G::kInstK + kWaves - 1) / kWaves;
  constexpr int kCopyV = (G::kInstV + kWaves - 1) / kWaves;
  int voff_k[kCopyK], voff_v[kCopyV];
#pragma unroll
  for (int k = 0; k < kCopyK; ++k) {
    const int u = (wave + k * kWaves) * 64 + lane;
    const int chunk = u % G::kSlotsK;
    voff_k[k] = (u / G::kSlotsK) * G::kRowBytes + (chunk < G::kChunks ? chunk : 0) * 16;
  }
#pragma unroll
  for (int k = 0; k < kCopyV; ++k) {
    const int u = (wave + k * kWaves) * 64 + lane;
    const int chunk = u % G::kSlotsV;
    voff_v[k] = (u / G::kSlotsV) * G::kRowBytes + (chunk < G::kChunks ? chunk : 0) * 16;
  }
  // LDS byte offsets of the two rings
  const unsigned lds_k = __builtin_amdgcn_readfirstlane(lds_offset_of(smem));
  const unsigned lds_v = lds_k + kRing * G::kTileK;
  auto copy_tile = [&](const __bf16* src, int slot, int j, auto is_k) __attribute__((always_inline)) {
    constexpr bool K_TILE = decltype(is_k)::value;
    constexpr int kInst = K_TILE ? G::kInstK : G::kInstV;
    constexpr int kCopy = K_TILE ? kCopyK : kCopyV;
    const int key0 = j * kBc;
    const i32x4 r = raw_rsrc(src + (long long)key0 * D, min(kBc, N - key0) * G::kRowBytes);
    const unsigned base = (K_TILE ? lds_k + slot * G::kTileK : lds_v + slot * G::kTileV) + wave * 1024;
#pragma unroll
    for (int k = 0; k < kCopy; ++k) {
      if (wave + k * kWaves < kInst)
        copy16_to_lds(r, K_TILE ? voff_k[k] : voff_v[k], base + k * kWaves * 1024);
    }
  };
  // copy instructions this wave issues per K (V) tile
  const int n_copy_k = (G::kInstK - wave + kWaves - 1) / kWaves;
  const int n_copy_v = (G::kInstV - wave + kWaves - 1) / kWaves;

  // Per-lane LDS offsets within a tile; the rest of every operand address
  // is an immediate.  K operand (kb, s): row 32*kb + l32, columns
  // 16*s + 8*half .. +7.  V transposing read for (db, kb, h, u): lane i of
  // each 16-lane group points at key row (i / 4) of a 4-row slab and dcol
  // 4*(i % 4) of a 16-column slab; lane i then receives the 4 keys of one
  // dcol (lane % 32).
  const int k_lane = l32 * G::kStrideK + 16 * half;
  const int v_lane = (4 * half + ((lane & 15) >> 2)) * G::kStrideV + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
  // operand bases of key tile j (ring slot j % 3)
  auto kbase_of = [&](int j) __attribute__((always_inline)) { return opaque(k_lane + (int)(lds_k + (j % kRing) * G::kTileK)); };
  auto vbase_of = [&](int j) __attribute__((always_inline)) { return opaque(v_lane + (int)(lds_v + (j % kRing) * G::kTileV)); };

  f32x16 oacc[G::kDBlocks];
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  // Two score tiles and two packed probability tiles: while the
  // probabilities of tile j are formed from sacc[j % 2] into pk[j % 2], the
  // matrix core writes S_{j+1} into sacc[(j + 1) % 2] and reads P_{j-1}
  // from pk[(j - 1) % 2].
  f32x16 sacc[2][2];
  bf16x8 pk[2][2][2];
  float m = -1e30f;  // reference max of raw scores (finite start)
  float l = 0.f;     // running denominator over this lane's keys

  // ---- one pipeline stage --------------------------------------------------
  // NPV MFMAs of O^T += V^T P^T (V^T from the tile at vbase, P^T from
  // pk[PB]), then NS MFMAs of S^T = K Q^T (K from the tile at kbase, into
  // sacc[SB]).  If PROBS, the softmax step of score tile sacc[XB] runs
  // between the MFMAs: the row max (four chains), the lazy move of m (see
  // kRescaleThreshold), and per score one FMA, one exp2 and one add (plus
  // one bf16 pack per pair) into pk[XB], software-pipelined three deep so
  // that no instruction waits on the one before it.  Each MFMA step is
  // fenced, so this interleave is the one the hardware sees.  Operands are
  // read from LDS kAhead MFMAs ahead of their use.  Returns this lane's sum
  // of the tile's probabilities, the factor alpha that l and O^T must be
  // multiplied by, and whether m moved anywhere in the wave.
  struct StageOut { float rs, alpha; bool moved; };
  auto stage = [&](auto npv_c, auto ns_c, auto probs_c, auto pb_c, auto sb_c, auto xb_c,
                   int kbase, int vbase) __attribute__((always_inline)) {
    constexpr int NPV = decltype(npv_c)::value;
    constexpr int NS = decltype(ns_c)::value;
    constexpr bool PROBS = decltype(probs_c)::value;
    constexpr int PB = decltype(pb_c)::value, SB = decltype(sb_c)::value, XB = decltype(xb_c)::value;
    constexpr int kSteps = NPV + NS;
    // steps that reduce the row max, then steps that start the 32 scores
    constexpr int kMaxSteps = kSteps >= 32 ? 4 : 2;
    constexpr int kElSteps = kSteps > kMaxSteps ? kSteps - kMaxSteps : 1;
    // scores whose FMA is issued at step n: [e_lo(n), e_lo(n + 1))
    auto e_lo = [](int n) {
      const int k = n - kMaxSteps;
      return k <= 0 ? 0 : k >= kElSteps ? 32 : (32 * k + kElSteps - 1) / kElSteps;
    };
    constexpr int kLastStep = (kSteps > kMaxSteps ? kSteps : kMaxSteps + 1) + 1;  // last A step
    auto read = [&](int n) __attribute__((always_inline)) {
      if (n < NPV) {
        // MFMA n: O^T block n % kDBlocks, key step n / kDBlocks = (kb, h);
        // operand slot u of lane (l32, half) is key 8*(u/4) + 4*half + (u%4)
        // in both the P^T operand (accumulator elements 8h..8h+7) and V^T.
        const int db = n % G::kDBlocks, ks = n / G::kDBlocks;
        const int off = (32 * (ks >> 1) + 16 * (ks & 1)) * G::kStrideV + 64 * db;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_cptr)(size_t)(vbase + off));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(lds_cptr)(size_t)(vbase + off + 8 * G::kStrideV));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      // MFMA NPV + s: score block s % 2 (two independent chains), k-step s / 2
      const int s = n - NPV;
      return *(const __attribute__((address_space(3))) bf16x8*)(lds_cptr)(size_t)(kbase + 32 * (s & 1) * G::kStrideK + 32 * (s >> 1));
    };
    auto mfma = [&](int n, const bf16x8& a) __attribute__((always_inline)) {
      if (n < NPV) {
        const int db = n % G::kDBlocks, ks = n / G::kDBlocks;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[PB][ks >> 1][ks & 1], oacc[db], 0, 0, 0);
      } else {
        const int s = n - NPV, kb = s & 1, ks = s >> 1;
        sacc[SB][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], ks == 0 ? f32x16{} : sacc[SB][kb], 0, 0, 0);
      }
    };
    // softmax state
    float mx[4], mc = 0.f, alpha = 1.f;
    bool moved = false;
    float t[32], p[32];
    u32x4 w[2][2];
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    auto score = [&](int e) __attribute__((always_inline)) { return sacc[XB][e >> 4][e & 15]; };
    auto max_part = [&](int g) __attribute__((always_inline)) {  // scores [32g/kMaxSteps, 32(g+1)/kMaxSteps)
#pragma unroll
      for (int e = 32 * g / kMaxSteps; e < 32 * (g + 1) / kMaxSteps; e += 8)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          mx[r] = (g == 0 && e == 0) ? fmaxf(score(e + r), score(e + r + 4))
                                     : fmaxf(fmaxf(mx[r], score(e + r)), score(e + r + 4));
    };
    auto decide = [&]() __attribute__((always_inline)) {
      const float mt = max_halves(fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3])));
      moved = __builtin_amdgcn_ballot_w64((mt - m) * c > kRescaleThreshold) != 0;
      const float m_new = moved ? fmaxf(m, mt) : m;
      alpha = __builtin_amdgcn_exp2f((m - m_new) * c);
      m = m_new;
      mc = pin(m * c);
    };
    // (each result is pinned where it is computed: without that, the
    // instruction selector is free to gather all of them after the MFMAs)
    auto op_f = [&](int e) __attribute__((always_inline)) {
      t[e] = pin(fmaf(score(e), c, -mc));
    };
    auto op_x = [&](int e) __attribute__((always_inline)) {
      p[e] = pin(__builtin_amdgcn_exp2f(t[e]));
    };
    auto op_a = [&](int e) __attribute__((always_inline)) {
      part[e & 3] = pin(part[e & 3] + p[e]);
      if (e & 1) {
        const bf16x2 pp = {(__bf16)p[e - 1], (__bf16)p[e]};
        const int kb = e >> 4, i = e & 15;
        w[kb][i >> 3][(i & 7) >> 1] = pin(__builtin_bit_cast(unsigned, pp));
      }
    };
    auto valu_of_step = [&](int n) __attribute__((always_inline)) {
      if (n < kMaxSteps) max_part(n);
      if (n == kMaxSteps - 1) decide();
#pragma unroll
      for (int e = e_lo(n - 2); e < e_lo(n - 1); ++e) op_a(e);
#pragma unroll
      for (int e = e_lo(n - 1); e < e_lo(n); ++e) op_x(e);
#pragma unroll
      for (int e = e_lo(n); e < e_lo(n + 1); ++e) op_f(e);
    };

    bf16x8 op[kAhead];
#pragma unroll
    for (int n = 0; n < kAhead && n < kSteps; ++n) op[n] = read(n);
#pragma unroll
    for (int n = 0; n < kSteps; ++n) {
      const bf16x8 a = op[n % kAhead];
      if (n + kAhead < kSteps) op[n % kAhead] = read(n + kAhead);
      mfma(n, a);
      if (PROBS) valu_of_step(n);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (PROBS) {
      // drain the pipeline (and, without MFMAs, run the whole softmax step)
#pragma unroll
      for (int n = kSteps; n <= kLastStep; ++n) valu_of_step(n);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        pk[XB][kb][0] = __builtin_bit_cast(bf16x8, w[kb][0]);
        pk[XB][kb][1] = __builtin_bit_cast(bf16x8, w[kb][1]);
      }
    }
    StageOut r{(part[0] + part[1]) + (part[2] + part[3]), alpha, moved};
    return r;
  };

  // Mask of the scores of tile j (keys past N; causal: keys after the row).
  // Element i of block kb holds key 64*j + 32*kb + 8*(i/4) + 4*half + (i%4).
  auto apply_mask = [&](auto xb_c, int j) __attribute__((always_inline)) {
    constexpr int XB = decltype(xb_c)::value;
    const int key0 = j * kBc;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
        const bool vis = (key < N) && (!CAUSAL || key <= qrow);
        if (!vis) sacc[XB][kb][i] = -INFINITY;
      }
  };
  // l and O^T banked against the old m are moved to the new one (O^T after
  // the stage's own MFMAs into it; the branch is taken only when m moved).
  auto bank = [&](const StageOut& r) __attribute__((always_inline)) {
    l = fmaf(l, r.alpha, r.rs);
    if (r.moved) {
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= r.alpha;
    }
  };
  using Z = std::integral_constant<int, 0>;
  using O = std::integral_constant<int, 1>;
  using PvN = std::integral_constant<int, kNPv>;
  using SN = std::integral_constant<int, kNS>;
  using Yes = std::true_type;
  using No = std::false_type;

  // ---- iterations ------------------------------------------------------------
  // Iteration it reads K_{it+1} (for S_{it+1}) and V_{it-1} (for P_{it-1} V).
  // It starts with a workgroup barrier: every wave has finished iteration
  // it-1, so the ring slots of K_it and V_{it-2} are free, and (each wave
  // having first waited for its own copies issued up to iteration it-2)
  // K_{it+1} and V_{it-1} have landed.  After the barrier the wave copies
  // K_{it+3} and V_{it+1} into the free slots.  The prologue provides K_0,
  // K_1, K_2 and V_0.  Every wave runs n_tiles + 1 iterations; it computes
  // in iterations 0 .. n_w and only takes part in the barriers and copies
  // after that.
  auto issue = [&](int it) __attribute__((always_inline)) {
    if (it + 3 < n_tiles) copy_tile(kh, it % kRing, it + 3, Yes{});
    if (it + 1 < n_tiles) copy_tile(vh, (it + 1) % kRing, it + 1, No{});
  };
  auto in_flight = [&](int it) __attribute__((always_inline)) {
    return (it + 3 < n_tiles ? n_copy_k : 0) + (it + 1 < n_tiles ? n_copy_v : 0);
  };
  auto sync = [&](int it) __attribute__((always_inline)) {
    if (it >= 1) wait_vmem(in_flight(it - 1));
    __syncthreads();
    issue(it);
  };

  // ---- prologue ----------------------------------------------------------------
  copy_tile(kh, 0, 0, Yes{});
  copy_tile(vh, 0, 0, No{});
  if (n_tiles > 1) copy_tile(kh, 1, 1, Yes{});
  if (n_tiles > 2) copy_tile(kh, 2, 2, Yes{});
  wait_vmem(0);
  __syncthreads();

  int it = 0;
  if (n_w >= 1) {
    stage(Z{}, SN{}, No{}, Z{}, Z{}, Z{}, kbase_of(0), 0);  // S_0
    sync(0);
    // tile 0 (m starts at -1e30, so the first softmax step always moves it;
    // nothing is banked yet, so alpha = 0 is harmless)
    if (n_w == 1) {
      if (mask_last) apply_mask(Z{}, 0);
      bank(stage(Z{}, Z{}, Yes{}, Z{}, Z{}, Z{}, 0, 0));
    } else {
      bank(stage(Z{}, SN{}, Yes{}, Z{}, O{}, Z{}, kbase_of(1), 0));
    }
    it = 1;
    // steady state: P_{j-1} V, softmax step of tile j, S_{j+1}
    auto steady = [&](int j, auto xb_c) __attribute__((always_inline)) {
      constexpr int X = decltype(xb_c)::value;
      using Xc = std::integral_constant<int, X>;
      using Yc = std::integral_constant<int, 1 - X>;
      sync(j);
      bank(stage(PvN{}, SN{}, Yes{}, Yc{}, Yc{}, Xc{}, kbase_of(j + 1), vbase_of(j - 1)));
    };
    for (; it + 1 <= n_w - 2; it += 2) {
      steady(it, O{});
      steady(it + 1, Z{});
    }
    if (it <= n_w - 2) {
      steady(it, O{});
      ++it;
    }
    // last tile of this wave (it = n_w - 1 >= 1): P_{it-1} V and its softmax step
    auto last = [&](int j, auto xb_c) __attribute__((always_inline)) {
      constexpr int X = decltype(xb_c)::value;
      using Xc = std::integral_constant<int, X>;
      using Yc = std::integral_constant<int, 1 - X>;
      sync(j);
      if (mask_last) apply_mask(Xc{}, j);
      bank(stage(PvN{}, Z{}, Yes{}, Yc{}, Z{}, Xc{}, 0, vbase_of(j - 1)));
    };
    if (n_w >= 2) {
      if (it & 1) last(it, O{});
      else last(it, Z{});
      ++it;
    }
    // it = n_w: P_{n_w - 1} V
    sync(it);
    if ((n_w - 1) & 1)
      stage(PvN{}, Z{}, No{}, O{}, Z{}, Z{}, 0, vbase_of(it - 1));
    else
      stage(PvN{}, Z{}, No{}, Z{}, Z{}, Z{}, 0, vbase_of(it - 1));
    ++it;
  }
  for (; it <= n_tiles; ++it) sync(it);

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
