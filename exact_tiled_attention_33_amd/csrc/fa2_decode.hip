// Decoding from a paged key/value cache with one wavefront per (chunk,
// sequence, key/value head, block of 32 query rows): the wavefront holds
// 32 of the group's query rows (H/H_kv heads x n_q new tokens, at most 128
// in all) and streams the chunk's keys
// and values in 32-key tiles through its own double-buffered LDS ring, with
// no workgroup barrier; four such wavefronts share a workgroup (and a CU)
// and each keeps its next tile in flight.  Decoding reads every key and
// value once from HBM and does little arithmetic per byte, so the kernel is
// built to keep many independent reads in flight, not to keep the matrix
// cores busy.
//
// Source: papermap "FlashAttention-2" explainer, Chapter 03 ("The
// Downstream Story"): paged-KV decoding is among the kernels built on
// FlashAttention-2; Mishra, "Another use of mergeable statistics": a long
// context is cut into chunks whose (max, sum) statistics merge exactly.
//
// Per tile: S^T = K Q^T (D/16 MFMAs 32x32x16, lane = query, keys in the
// accumulator), the online softmax over the tile (max, rescale, exp2, two
// row sums: fp32 for LSE, of the bf16-rounded probabilities for O), then
// O^T += V^T P^T (2*D/32 MFMAs, V read transposed from LDS).  Each chunk
// writes a partial result in the layout of the paged kernel; the same merge
// kernel combines them.

#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "fa2.h"
#include "fa2_launch.h"

// Partial results of fa2_decode_paged_noalloc.  The runtime gives every
// device its own copy, kept until the process ends.  In host code this name
// stands for the variable, not a device address: only the per-device address
// that decode_scratch() looks up may be handed to a kernel or a copy.
static __device__ __align__(256) unsigned char scratch[FA2_DECODE_SCRATCH_BYTES];

namespace fa2 {

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> by_device[kMaxDevices];
  static std::mutex lookup;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = by_device[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> g(lookup);
    p = by_device[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      by_device[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kDecWaves = 4;   // independent wavefronts per workgroup
constexpr int kDecKeys = 32;   // keys per tile
constexpr int kDecStages = 2;  // tiles resident per wavefront (one in flight while one is used)

template <int D>
struct DecGeo {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kStrideK = kRowBytes + 16;  // conflict-free 16-byte operand reads (as the forward kernel)
  // V rows unpadded, their 64-byte units XOR-permuted by vswz(row) (as the
  // forward kernel): conflict-free transposing reads
  static constexpr int kStrideV = kRowBytes;
  static constexpr int kSlotsK = kStrideK / 16;
  static constexpr int kSlotsV = kStrideV / 16;
  static __device__ __forceinline__ int vswz(int r) { return D == 128 ? (r & 3) : ((r >> 1) & 1); }
  static constexpr int kChunks = kRowBytes / 16;   // data chunks per row
  // copy instructions per tile (64 lanes x 16 bytes each); the last K
  // instruction may cover slots past the tile, which land in padding
  static constexpr int kInstK = (kDecKeys * kSlotsK + 63) / 64;
  static constexpr int kInstV = (kDecKeys * kSlotsV + 63) / 64;
  static constexpr int kBytesK = kInstK * 1024;
  static constexpr int kBytesV = kInstV * 1024;
  static constexpr int kStage = kBytesK + kBytesV;
  static constexpr int kWaveLds = kDecStages * kStage;
  static constexpr int kKSteps = D / 16;
  static constexpr int kDBlocks = D / 32;
};

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// 16 bytes per lane from global memory (wave-uniform base, per-lane
// offset) straight into LDS at lds_offset + 16*lane.
__device__ __forceinline__ void dec_copy16(unsigned long long base, int voff, unsigned lds_offset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_offset), "v"(voff), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

// Waits for a loaded value before the next tile copy is issued.  The
// compiler cannot see the copies (inline asm), so to it a register load
// stays the newest vector-memory operation: a use of it inside the tile
// loop would get a vmcnt(0) wait, which in hardware also drains the tile
// in flight -- on every tile.  Using the value here, in an asm statement
// that stays ordered before the copies and redefines it, puts that wait
// once before the copies instead.
template <typename T>
__device__ __forceinline__ void dec_landed(T& x) {
  asm volatile("" : "+v"(x));
}

__device__ __forceinline__ unsigned long long dec_uniform(const void* p) {
  const unsigned long long b = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(b & 0xffffffffu));
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// s_waitcnt with vmcnt <= N (0..63), the other counters left alone.
template <int N>
__device__ __forceinline__ void dec_wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ float dec_max_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float dec_sum_halves(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

template <int D>
__global__ __launch_bounds__(64 * kDecWaves) void decode_wave_kernel(const __bf16* __restrict__ q,
                                                                     const __bf16* __restrict__ kc,
                                                                     const __bf16* __restrict__ vc,
                                                                     float* __restrict__ part, PagedArgs pg,
                                                                     int groups, int n_waves, int nq_rows,
                                                                     int n_slots, int max_keys, int group, float c) {
  using G = DecGeo<D>;
  __shared__ __attribute__((aligned(1024))) char smem[kDecWaves * G::kWaveLds];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // this wavefront's (chunk, group, row block); the row blocks of a group
  // are adjacent wavefronts, so a workgroup's wavefronts read the same pages
  const int gw = blockIdx.x * kDecWaves + w;
  if (gw >= n_waves) return;  // whole wavefronts only; no barrier in this kernel
  const int n_rb = (nq_rows + 31) / 32, rb = gw % n_rb;
  const int g = (gw / n_rb) % groups, chunk = gw / n_rb / groups;
  const int b = g / pg.kv_heads, kvh = g % pg.kv_heads;
  const int n_keys = min(min(max(pg.ctx_lens[b], 0), pg.max_pages * pg.page_size), max_keys);
  const int key_begin = chunk * pg.chunk_tiles * 64;
  if (key_begin >= n_keys) return;  // chunk past this sequence's context
  const int key_end = min(key_begin + pg.chunk_tiles * 64, n_keys);
  const int t0 = key_begin / kDecKeys, nt = (key_end - key_begin + kDecKeys - 1) / kDecKeys;
  const int* const page_row = pg.page_table + (long long)b * pg.max_pages;
  const int l32 = lane & 31, half = lane >> 5;
  const int qrow = 32 * rb + l32;  // this lane's query row within the group

  // The row block's Q rows as MFMA B operands (query = lane % 32, dims
  // 16*s + 8*half .. +7); rows past nq_rows read as zeros.
  bf16x8 qf[G::kKSteps];
  {
    const __bf16* qg = q + ((long long)g * nq_rows + 32 * rb) * D;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16*>(qg), (short)0, __builtin_amdgcn_readfirstlane(min(32, nq_rows - 32 * rb) * D * 2),
        0x00020000);
#pragma unroll
    for (int s = 0; s < G::kKSteps; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                        rq, (l32 * D + 16 * s + 8 * half) * 2, 0, 0)));
  }

  const unsigned lds_wave = __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(const __attribute__((address_space(3))) char*)smem) + w * G::kWaveLds;
  const char* const lds_wave_ptr = smem + w * G::kWaveLds;
  const int row_bytes = pg.kv_heads * G::kRowBytes;  // bytes between consecutive keys in the cache

  // The chunk's page numbers, one per lane for 64 pages at a time: a tile
  // takes its page with a lane read, not a load.  Tiles never straddle
  // pages (pages hold a multiple of 64 keys), so the page number grows by
  // at most one per tile and a new window is loaded once per 64 pages.
  int page_base = key_begin / pg.page_size;
  int page_lane = page_row[min(page_base + lane, pg.max_pages - 1)];
  auto page_of = [&](int key0) __attribute__((always_inline)) {
    const int pi = key0 / pg.page_size;
    if (pi - page_base >= 64) {
      page_base += 64;
      page_lane = page_row[min(page_base + lane, pg.max_pages - 1)];
      dec_landed(page_lane);
    }
    return min(max(__builtin_amdgcn_readlane(page_lane, pi - page_base), 0), pg.n_pages - 1);
  };
  dec_landed(page_lane);
#pragma unroll
  for (int s = 0; s < G::kKSteps; ++s) dec_landed(qf[s]);

  // Copy tile i (keys key0 .. key0 + 31 of this chunk) into stage st.
  auto copy_tile = [&](int i, int st) __attribute__((always_inline)) {
    const int key0 = (t0 + i) * kDecKeys;
    const int rows = min(kDecKeys, n_keys - key0);
    const int page = page_of(key0);
    const long long off = (((long long)page * pg.page_size + key0 % pg.page_size) * pg.kv_heads + kvh) * D;
    const unsigned long long gk = dec_uniform(kc + off), gv = dec_uniform(vc + off);
    const unsigned base = lds_wave + st * G::kStage;
#pragma unroll
    for (int k = 0; k < G::kInstK; ++k) {
      const int u = 64 * k + lane, chunk = u % G::kSlotsK;
      const int r = min(u / G::kSlotsK, rows - 1);  // slots past the tile or the context fetch a valid row
      dec_copy16(gk, r * row_bytes + (chunk < G::kChunks ? chunk : 0) * 16, base + 1024 * k);
    }
#pragma unroll
    for (int k = 0; k < G::kInstV; ++k) {
      // slot u: LDS row u / kChunks, stored chunk u % kChunks = the row's
      // chunk (u % kChunks) ^ 4*vswz(row)
      const int u = 64 * k + lane, row = u / G::kSlotsV;
      const int chunk = (u % G::kSlotsV) ^ (4 * G::vswz(row));
      const int r = min(row, rows - 1);
      dec_copy16(gv, r * row_bytes + chunk * 16, base + G::kBytesK + 1024 * k);
    }
  };

  // operand offsets (as the forward kernel, one 32-key block per tile)
  const int k_lane = l32 * G::kStrideK + 16 * half;
  // V: the lane's row within each 8-row slab is 4*half + (lane%16)/4; its
  // 64-byte unit db is stored at unit db ^ vswz(row)
  const int v_row = 4 * half + ((lane & 15) >> 2);
  int v_lane[G::kDBlocks];
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
    v_lane[db] = v_row * G::kStrideV + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2 + 64 * (db ^ G::vswz(v_row));

  f32x16 oacc[G::kDBlocks];
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m = -INFINITY;  // running max of raw scores
  float l = 0.f, lb = 0.f;
  // new token i of n_q sits at position n_keys - n_q + i and sees keys up to it
  const int key_hi = n_keys - pg.n_q + qrow % pg.n_q;
  const int full_hi = n_keys - pg.n_q;  // keys every row sees: <= full_hi
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Tile i sits in stage i % 2.  Iteration i first copies tile i+1 into
  // the stage of tile i-1 (whose reads all fed iteration i-1's MFMAs), then
  // waits until tile i has landed, leaving tile i+1 in flight.  (Three
  // wavefronts with 3-stage rings, two tiles in flight each, moved less:
  // 3.4 TB/s against 4.1.)
  copy_tile(0, 0);
  int st = 0;
  for (int i = 0; i < nt; ++i) {
    if (i + 1 < nt) {
      copy_tile(i + 1, st ^ 1);
      dec_wait_vmem<G::kInstK + G::kInstV>();
    } else {
      dec_wait_vmem<0>();
    }
    const char* kbuf = lds_wave_ptr + st * G::kStage;
    const char* vbuf = kbuf + G::kBytesK;
    f32x16 sacc = {};
#pragma unroll
    for (int s = 0; s < G::kKSteps; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kbuf + k_lane + 32 * s), qf[s], sacc, 0, 0, 0);
    // element e holds key key0 + 8*(e/4) + 4*half + (e%4)
    const int key0 = (t0 + i) * kDecKeys;
    if (key0 + kDecKeys - 1 > full_hi) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = key0 + 8 * (e >> 2) + 4 * half + (e & 3);
        sacc[e] = key <= key_hi ? sacc[e] : -INFINITY;
      }
    }
    float mt = sacc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) mt = fmaxf(mt, sacc[e]);
    mt = dec_max_halves(mt);
    const float m_new = fmaxf(m, mt);
    const float ref = m_new > -INFINITY ? m_new : 0.f;  // no visible key yet: probabilities are 0
    const float alpha = m > -INFINITY ? exp2f((m - ref) * c) : 0.f;
    m = m_new;
    float ps = 0.f, pbs = 0.f;
    bf16x8 pk[2];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[e], c, -ref * c));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[e + 1], c, -ref * c));
      ps += p0 + p1;
      const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
      pbs = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, pbs, false);
      pk[e >> 3][e & 7] = pp[0];
      pk[e >> 3][(e & 7) + 1] = pp[1];
    }
    l = l * alpha + ps;
    lb = lb * alpha + pbs;
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    // O^T += V^T P^T: key step h covers keys 16h .. 16h+15 of the tile
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db) {
        const int off = v_lane[db] + (16 * h) * G::kStrideV;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbuf + off));
        const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(vbuf + off + 8 * G::kStrideV));
        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk[h], oacc[db], 0, 0, 0);
      }
    st ^= 1;
  }

  // partial result of the chunk (layout of the paged kernel's partials)
  const float lt = dec_sum_halves(l), ltb = dec_sum_halves(lb);
  if (qrow >= nq_rows) return;
  const float inv = ltb > 0.f ? 1.0f / ltb : 0.f;
  float* const po = part + (((long long)g * n_slots + chunk) * nq_rows + qrow) * D;
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4)
      *(float4*)(po + 32 * db + 8 * a4 + 4 * half) =
          make_float4(oacc[db][4 * a4] * inv, oacc[db][4 * a4 + 1] * inv, oacc[db][4 * a4 + 2] * inv,
                      oacc[db][4 * a4 + 3] * inv);
  if (half == 0) {
    float2* const pl = (float2*)(part + (long long)groups * n_slots * nq_rows * D) +
                       ((long long)g * n_slots + chunk) * nq_rows + qrow;
    *pl = make_float2(lt > 0.f ? (m * c + log2f(lt)) * 0.69314718055994531f : -INFINITY,
                      ltb > 0.f ? (m * c + log2f(ltb)) * 0.69314718055994531f : -INFINITY);
  }
}

template <int D>
hipError_t launch_wave_d(const FwdArgs& a) {
  const int groups = a.B * a.Hkv;
  const int nq_rows = (a.H / a.Hkv) * a.paged.n_q;
  const long long n_waves = (long long)a.n_slots * groups * ((nq_rows + 31) / 32);
  const long long grid = (n_waves + kDecWaves - 1) / kDecWaves;
  if (n_waves > 0x7fffffffLL || grid < 1) return hipErrorInvalidValue;
  const float c = fmaxf(a.scale * 1.4426950408889634f, 1e-30f);
  hipLaunchKernelGGL((decode_wave_kernel<D>), dim3((unsigned)grid), dim3(64 * kDecWaves), 0, a.stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (float*)a.part, a.paged, groups,
                     (int)n_waves, nq_rows, a.n_slots, a.N, a.H / a.Hkv, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_waves(const FwdArgs& a) {
  switch (a.d) {
    case 64: return launch_wave_d<64>(a);
    case 128: return launch_wave_d<128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa2
