// Internal interface between the C-ABI front end (fa2_api.cpp) and the
// kernel translation units.  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

namespace fa2 {

// One chunk of a split forward schedule (the layout of fa2_split_item in
// fa2.h): query tile `tile`, key tiles [kt_lo, kt_hi) of it; `slot` is the
// partial-result slot (-1: the chunk is the whole tile and writes O and LSE
// itself); the tile's chunks use slots slot0 .. slot0 + n_parts - 1.
struct SplitItem {
  int tile, kt_lo, kt_hi, slot, slot0, n_parts;
};

// Paged key/value cache of a decoding call: caches [n_pages][page_size]
// [kv_heads][d]; logical key j of sequence b is in page
// page_table[b*max_pages + j/page_size], slot j % page_size.  Each
// workgroup takes chunk_tiles key tiles of one (sequence, key/value head).
struct PagedArgs {
  const int* page_table = nullptr;
  const int* ctx_lens = nullptr;
  int max_pages = 0;
  int page_size = 0;
  int n_pages = 0;
  int n_q = 1;
  int chunk_tiles = 1;
  int kv_heads = 1;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H, N, d;
  int Hkv;  // key/value heads (H for ordinary multi-head attention)
  bool causal;
  // Sliding window: key j visible to query i iff i - wl <= j <= i + wr; -1 =
  // no limit on that side (causal: wl = -1, wr = 0; none: both -1).
  int wl, wr;
  float scale;
  bool o_bf16;
  // Debug: fill each LDS ring slot with NaN before a tile is copied into it
  // (bf16 kernel; set from the FA2_DEBUG_POISON environment variable).
  bool poison;
  // Split schedule (bf16 kernel): device array of n_items chunks, or null
  // for one workgroup per query tile; partial results go to `part`
  // (n_slots slots per (batch, head)).
  const void* items = nullptr;
  int n_items = 0;
  void* part = nullptr;
  int n_slots = 0;
  // Block-sparse list (bf16 kernel): per (layout, query tile) offsets
  // sp_ptr[n_layouts*T + 1] into the entries sp_ent[n_entries]; layout of
  // (b, h) = (b*H + h) % n_layouts.  Null: dense.
  const int* sp_ptr = nullptr;
  const unsigned* sp_ent = nullptr;
  int n_layouts = 1;
  int n_entries = 0;
  // Paged decoding (launch_decode_paged): n_q new tokens per sequence, N =
  // the largest context; n_slots = chunks per (sequence, key/value head).
  PagedArgs paged;
  // FP8 forward (bf16 kernel's FP8 mode): q and k hold E4M3 codes, one fp32
  // scale per (b, h) in q_scale[B*H] and per (b, kv head) in k_scale.
  bool fp8 = false;
  const float* q_scale = nullptr;
  const float* k_scale = nullptr;
  hipStream_t stream;
};

// Tile geometry of each kernel family.  The bf16 kernel gives every
// wavefront 32 query rows (the N side of a 32x32 MFMA) and streams keys in
// tiles of kBf16BlockCols; the fp32 kernel does the same with 32-key tiles.
constexpr int kBf16Waves = 8;
constexpr int kBf16BlockRows = kBf16Waves * 32;  // 256
constexpr int kBf16BlockCols = 64;
// The forward kernel of fa2_fwd / fa2_fwd_gqa / fa2_fwd_window (bf16 in):
// workgroups of 4 wavefronts x 32 rows, two per compute unit, the same
// 64-key tiles.  (The 256-row geometry above serves the split, block-sparse,
// paged and FP8 modes.)
constexpr int kFwdWaves = 4;
constexpr int kFwdBlockRows = kFwdWaves * 32;  // 128

// How that kernel's items ((query tile, batch*head) pairs) go to workgroups,
// two of which fit a compute unit.  sched 0: one item per workgroup (the
// hardware hands out items as units free up); 1: equal items in rounds,
// workgroup g taking g, g + G, ... (G a multiple of 8, so that a workgroup
// keeps to one XCD's items) when there are more than the units hold at
// once (used at d = 64, where it measured faster; at d = 128 the loop
// over items costs the kernel registers it does not have to spare); 2:
// items of growing length (a causal mask or a window open to the left),
// more than one per unit but at most two: G = ceil(items / 2) workgroups
// each take the i-th heaviest and the i-th lightest item.
struct FwdSchedule {
  long long workgroups;
  int sched;
};
inline FwdSchedule fwd_schedule(long long items, int units, bool uneven, int d) {
  const long long slots = 2LL * units;
  if (!uneven && d == 64 && items > slots) {
    const long long rounds = (items + slots - 1) / slots;
    long long groups = (items + rounds - 1) / rounds;
    groups = (groups + 7) / 8 * 8;
    return {groups, 1};
  }
  if (uneven && items > units && items <= slots) return {(items + 1) / 2, 2};
  return {items, 0};
}
constexpr int kF32Waves = 4;
constexpr int kF32BlockRows = kF32Waves * 32;    // 128
constexpr int kF32BlockCols = 32;

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;
  void* dq;
  void* dk;
  void* dv;
  int B, H, N, d;
  int Hkv;  // key/value heads (H for ordinary multi-head attention)
  bool causal;
  int wl, wr;  // sliding window, as in FwdArgs
  float scale;
  bool o_bf16;
  bool grad_bf16;
  hipStream_t stream;
};

// Backward tile geometry (bf16 inputs): the dQ kernel gives each of its
// kBwdQWaves wavefronts 32 query rows and streams 64-key tiles; the dK/dV
// kernel gives each wavefront of a group 32 keys (kBwdKVKeys per
// workgroup) and streams 32-query blocks, the two groups taking alternate
// blocks.
constexpr int kBwdQWaves = 8;
constexpr int kBwdQRows = kBwdQWaves * 32;  // 256
constexpr int kBwdQCols = 64;
constexpr int kBwdKVKeys = 128;
constexpr int kBwdKVRows = 32;

// Signs of the FP8 rotation: bit i set = coordinate i negated (d <= 128).
struct Fp8Signs {
  unsigned bits[4];
};

// FP8 packing of one [BH][N][d] bf16 tensor (fa2_fp8.hip).
struct Fp8PackArgs {
  const void* x;
  int BH, N, d;
  bool rotate;
  Fp8Signs signs;
  void* codes;      // [BH][N][d] E4M3 codes
  float* scales;    // [BH]
  float* partial;   // workspace: [BH][fp8_pack_chunks(N)] chunk maxima
  hipStream_t stream;
};

int fp8_pack_chunks(int N);
hipError_t launch_fp8_pack(const Fp8PackArgs& a);

// Enqueue the merge of split partial results into O and LSE (after the
// forward kernel, on the same stream).
hipError_t launch_split_merge(const FwdArgs& a);

// Enqueue paged decoding: the chunk kernel, then the merge of its partials.
hipError_t launch_decode_paged(const FwdArgs& a);
// Device address of the static decode scratch (FA2_DECODE_SCRATCH_BYTES) on
// the current device, looked up once per device.
hipError_t decode_scratch(void** ptr);

// The chunk kernel of paged decoding with one wavefront per (chunk, group)
// (fa2_decode.hip), for groups of at most 32 query rows.
hipError_t launch_decode_waves(const FwdArgs& a);

// Enqueue the backward kernels (D, dK/dV, dQ) for bf16 inputs.
hipError_t launch_bwd_bf16(const BwdArgs& a);

// Enqueue the forward kernel for bf16 (resp. fp32) inputs.  Arguments are
// already validated; returns the launch status.
hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);

}  // namespace fa2
