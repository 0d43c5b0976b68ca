// C-ABI front end: argument validation, launch geometry, dispatch.
//
// Every check runs before the first HIP call, so malformed calls are
// rejected identically on machines with and without a GPU.

#include "fa2.h"

#include <algorithm>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <functional>
#include <queue>
#include <vector>

#include "fa2_launch.h"

#include <cstdlib>

namespace {

bool is_dtype(int x) { return x == FA2_F32 || x == FA2_BF16; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [p, p + n) and [q, q + m) share a byte?
bool overlaps(const void* p, size_t n, const void* q, size_t m) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

int check_sizes(int B, int H, int N, int d, int in_dtype) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA2_ERR_INVALID_ARG;
  if (!is_dtype(in_dtype)) return FA2_ERR_INVALID_ARG;
  // B*H*N*d elements (and bytes) must fit comfortably in 64-bit offsets.
  const long double elems = (long double)B * H * N * d;
  if (elems > (long double)(1LL << 60)) return FA2_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA2_ERR_UNSUPPORTED;
  return FA2_OK;
}

void own_tiles(int in_dtype, int* rows, int* cols, int* waves) {
  if (in_dtype == FA2_BF16) {
    *rows = fa2::kFwdBlockRows; *cols = fa2::kBf16BlockCols; *waves = fa2::kFwdWaves;
  } else {
    *rows = fa2::kF32BlockRows; *cols = fa2::kF32BlockCols; *waves = fa2::kF32Waves;
  }
}

// Validation shared by the forward entry points; fills *a on success.
int prepare_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N,
                int d, int window_left, int window_right, float scale, void* stream, int in_dtype, int o_dtype,
                fa2::FwdArgs* a) {
  if (!q || !k || !v || !o || !lse) return FA2_ERR_INVALID_ARG;
  if (window_left < -1 || window_right < -1) return FA2_ERR_INVALID_ARG;
  if (H_kv < 1 || H < 1 || H % H_kv != 0) return FA2_ERR_INVALID_ARG;
  if (!is_dtype(o_dtype)) return FA2_ERR_INVALID_ARG;
  const int st = check_sizes(B, H, N, d, in_dtype);
  if (st != FA2_OK) return st;
  // a bound of N or more keys is no bound (this also keeps the kernels'
  // index arithmetic in range)
  const int wl = window_left >= N ? -1 : window_left;
  const int wr = window_right >= N ? -1 : window_right;
  const bool causal = (wl == -1 && wr == 0);
  // the fp32 kernel implements no mask and the causal mask only
  if (in_dtype == FA2_F32 && !(wl == -1 && (wr == -1 || wr == 0))) return FA2_ERR_UNSUPPORTED;
  if (!std::isfinite(scale) || scale < 0.f) return FA2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA2_ERR_INVALID_ARG;
  const size_t elems = (size_t)B * H * N * d;
  const size_t esz = in_dtype == FA2_BF16 ? 2 : 4;
  const size_t q_bytes = elems * esz;
  const size_t kv_bytes = (size_t)B * H_kv * N * d * esz;
  const size_t o_bytes = elems * (o_dtype == FA2_BF16 ? 2 : 4);
  const size_t lse_bytes = (size_t)B * H * N * sizeof(float);
  const void* ins[3] = {q, k, v};
  const size_t in_sz[3] = {q_bytes, kv_bytes, kv_bytes};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(o, o_bytes, ins[i], in_sz[i]) || overlaps(lse, lse_bytes, ins[i], in_sz[i]))
      return FA2_ERR_INVALID_ARG;
  }
  if (overlaps(o, o_bytes, lse, lse_bytes)) return FA2_ERR_INVALID_ARG;

  a->q = q; a->k = k; a->v = v; a->o = o; a->lse = lse;
  a->B = B; a->H = H; a->N = N; a->d = d;
  a->Hkv = H_kv;
  a->causal = causal;
  a->wl = wl;
  a->wr = wr;
  a->scale = scale;
  a->o_bf16 = (o_dtype == FA2_BF16);
  const char* dbg = std::getenv("FA2_DEBUG_POISON");
  a->poison = dbg != nullptr && dbg[0] != '\0' && dbg[0] != '0';
  a->stream = reinterpret_cast<hipStream_t>(stream);
  return FA2_OK;
}

// ---- split schedules ----------------------------------------------------------
static_assert(sizeof(fa2_split_item) == sizeof(fa2::SplitItem), "fa2_split_item and SplitItem must match");
static_assert(offsetof(fa2_split_item, n_parts) == offsetof(fa2::SplitItem, n_parts), "layout mismatch");

// Cost model of the bf16 forward kernel in units of one key-tile step of
// one workgroup: the fixed cost of a workgroup (its Q rows, the first
// copies, the epilogue), the HBM cost of writing and re-reading one partial
// result (256 rows x (d fp32 + 2 log-sums), about 0.07 us at 4 TB/s against
// about 2 us per key-tile step at d = 128; both scale with d), and the
// merge kernel's launch.
constexpr double kItemSteps = 2.0;
constexpr double kPartialSteps = 0.035;
constexpr double kMergeLaunchSteps = 2.0;
// split only when the model predicts at least this gain
constexpr double kSplitMinGain = 0.95;
constexpr int kMinChunkTiles = 2;

struct KeyRange {
  int tile, lo, hi;  // key tiles [lo, hi) visible to some row of the tile
};

// The key tiles the bf16 kernel streams for each query tile under the
// window (the same band rule as the kernel).
std::vector<KeyRange> key_ranges(int N, int wl, int wr) {
  const int br = fa2::kBf16BlockRows, bc = fa2::kBf16BlockCols;
  const int T = (N + br - 1) / br, nk = (N + bc - 1) / bc;
  std::vector<KeyRange> out((size_t)T);
  for (int t = 0; t < T; ++t) {
    const int q0 = t * br, q_last = std::min(q0 + br, N) - 1;
    const int lo = wl >= 0 ? std::max(0, q0 - wl) / bc : 0;
    const int hi = wr >= 0 ? std::min(nk, (q_last + wr) / bc + 1) : nk;
    out[(size_t)t] = {t, lo, hi};
  }
  return out;
}

// Cut every range of more than `chunk` key tiles (0: none) into equal
// chunks; list them longest first.  Returns the number of partial slots.
int make_schedule(const std::vector<KeyRange>& ranges, int chunk, std::vector<fa2_split_item>* out) {
  out->clear();
  int slots = 0;
  for (const KeyRange& r : ranges) {
    const int n = r.hi - r.lo;
    const int parts = (chunk > 0 && n > chunk) ? (n + chunk - 1) / chunk : 1;
    for (int p = 0; p < parts; ++p) {
      fa2_split_item it;
      it.tile = r.tile;
      it.kt_lo = r.lo + (int)((long long)n * p / parts);
      it.kt_hi = r.lo + (int)((long long)n * (p + 1) / parts);
      it.slot = parts > 1 ? slots + p : -1;
      it.slot0 = parts > 1 ? slots : -1;
      it.n_parts = parts;
      out->push_back(it);
    }
    if (parts > 1) slots += parts;
  }
  std::stable_sort(out->begin(), out->end(), [](const fa2_split_item& a, const fa2_split_item& b) {
    const int na = a.kt_hi - a.kt_lo, nb = b.kt_hi - b.kt_lo;
    if (na != nb) return na > nb;
    return a.tile > b.tile;
  });
  return slots;
}

// Predicted duration of a schedule: the workgroups (item-major, B*H per
// item) go in grid order to whichever unit frees first; plus the partial
// traffic and the merge.
double schedule_cost(const std::vector<fa2_split_item>& items, int slots, long long bh, int units) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int u = 0; u < units; ++u) free_at.push(0.0);
  double end = 0.0;
  for (const fa2_split_item& it : items) {
    const double cost = kItemSteps + (it.kt_hi - it.kt_lo);
    for (long long h = 0; h < bh; ++h) {
      const double t0 = free_at.top();
      free_at.pop();
      free_at.push(t0 + cost);
      end = std::max(end, t0 + cost);
    }
  }
  if (slots > 0) end += kMergeLaunchSteps + kPartialSteps * (double)slots * (double)bh;
  return end;
}

size_t split_workspace_bytes(int B, int H, int d, int slots) {
  return (size_t)B * H * slots * fa2::kBf16BlockRows * ((size_t)d * sizeof(float) + 2 * sizeof(float));
}

}  // namespace

extern "C" {

int fa2_version(void) { return FA2_VERSION; }

const char* fa2_strerror(int status) {
  switch (status) {
    case FA2_OK: return "success";
    case FA2_ERR_INVALID_ARG: return "invalid argument (null/misaligned/overlapping pointer, bad size, scale or dtype code)";
    case FA2_ERR_UNSUPPORTED: return "unsupported configuration (head dim 64 or 128; backward: bf16 inputs)";
    case FA2_ERR_NO_DEVICE: return "no HIP device available";
    case FA2_ERR_LAUNCH: return "kernel launch failed";
    case FA2_ERR_SCRATCH: return "the call needs more than the static scratch of a no-alloc entry point";
    default: return "unknown status";
  }
}

int fa2_plan(int B, int H, int N, int d, int causal, int in_dtype, int block_rows, int block_cols,
             int num_units, fa2_plan_t* out) {
  if (out == nullptr) return FA2_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARG;
  if (block_rows < 0 || block_cols < 0 || num_units < 0) return FA2_ERR_INVALID_ARG;
  const int st = check_sizes(B, H, N, d, in_dtype);
  if (st != FA2_OK) return st;

  int br, bc, waves;
  own_tiles(in_dtype, &br, &bc, &waves);
  if (block_rows > 0) br = block_rows;
  if (block_cols > 0) bc = block_cols;

  const long long bh = (long long)B * H;
  const long long T = (N + (long long)br - 1) / br;
  const long long nk = (N + (long long)bc - 1) / bc;
  // Key tiles visited per query tile: all of them, or (causal) those that
  // start at or below the tile's last row.
  long long pairs_per_head = 0;
  for (long long t = 0; t < T; ++t) {
    if (!causal) {
      pairs_per_head += nk;
    } else {
      const long long last_row = std::min<long long>((t + 1) * br - 1, (long long)N - 1);
      pairs_per_head += std::min<long long>(nk, last_row / bc + 1);
    }
  }
  out->block_rows = br;
  out->block_cols = bc;
  out->waves_per_group = waves;
  out->query_tiles = (int)T;
  out->workgroups = bh * T;
  out->tile_pairs = bh * pairs_per_head;
  out->normalisations = bh * T;
  out->waves_of_groups = num_units > 0 ? (double)out->workgroups / num_units : 0.0;
  out->last_wave_groups = num_units > 0 ? (int)(out->workgroups % num_units) : 0;
  out->flops_executed = 4.0 * (double)br * bc * d * (double)out->tile_pairs;
  out->flops_credited = 4.0 * (double)bh * N * (double)N * d / (causal ? 2.0 : 1.0);
  return FA2_OK;
}

int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
            int d, int causal, float scale, void* stream, int in_dtype, int o_dtype) {
  return fa2_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, stream, in_dtype, o_dtype);
}

int fa2_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int H_kv, int N, int d, int causal, float scale, void* stream, int in_dtype,
                int o_dtype) {
  if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARG;
  return fa2_fwd_window(q, k, v, o, lse, B, H, H_kv, N, d, -1, causal ? 0 : -1, scale, stream, in_dtype,
                        o_dtype);
}

int fa2_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int H_kv, int N, int d, int window_left, int window_right, float scale, void* stream,
                   int in_dtype, int o_dtype) {
  fa2::FwdArgs a;
  const int st = prepare_fwd(q, k, v, o, lse, B, H, H_kv, N, d, window_left, window_right, scale, stream,
                             in_dtype, o_dtype, &a);
  if (st != FA2_OK) return st;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA2_ERR_NO_DEVICE;
  const hipError_t e = (in_dtype == FA2_BF16) ? fa2::launch_fwd_bf16(a) : fa2::launch_fwd_f32(a);
  return e == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

int fa2_split_plan(int B, int H, int N, int d, int window_left, int window_right, int in_dtype,
                   int num_units, int max_chunk_tiles, fa2_split_item* items, int max_items, int* n_items,
                   int* n_slots, size_t* workspace_bytes) {
  if (!n_items || !n_slots || !workspace_bytes) return FA2_ERR_INVALID_ARG;
  if (window_left < -1 || window_right < -1 || max_chunk_tiles < 0 || max_items < 0) return FA2_ERR_INVALID_ARG;
  if (max_chunk_tiles == 0 && num_units < 1) return FA2_ERR_INVALID_ARG;
  const int st = check_sizes(B, H, N, d, in_dtype);
  if (st != FA2_OK) return st;
  if (in_dtype != FA2_BF16) return FA2_ERR_UNSUPPORTED;
  const int wl = window_left >= N ? -1 : window_left;
  const int wr = window_right >= N ? -1 : window_right;
  const std::vector<KeyRange> ranges = key_ranges(N, wl, wr);
  const long long bh = (long long)B * H;
  std::vector<fa2_split_item> plan;
  int slots = 0;
  if (max_chunk_tiles > 0) {
    slots = make_schedule(ranges, max_chunk_tiles, &plan);
  } else {
    // candidates: no split; chunks of about total / (k * units) key tiles
    // (k workgroups per unit); and chunks that cut the longest band into s
    // equal parts
    slots = make_schedule(ranges, 0, &plan);
    const double whole = schedule_cost(plan, slots, bh, num_units);
    long long total = 0, longest = 0;
    for (const KeyRange& r : ranges) {
      total += r.hi - r.lo;
      longest = std::max<long long>(longest, r.hi - r.lo);
    }
    total *= bh;
    std::vector<long long> chunks;
    for (int k4 : {4, 5, 6, 7, 8, 10, 12, 16, 24, 32}) {  // k = k4 / 4
      chunks.push_back((4 * total + (long long)k4 * num_units - 1) / ((long long)k4 * num_units));
    }
    for (int parts = 2; parts <= 8; ++parts) chunks.push_back((longest + parts - 1) / parts);
    std::sort(chunks.begin(), chunks.end());
    chunks.erase(std::unique(chunks.begin(), chunks.end()), chunks.end());
    double best = whole * kSplitMinGain;
    for (const long long c0 : chunks) {
      const long long c = std::max<long long>(kMinChunkTiles, c0);
      if (c > (1 << 30)) continue;
      std::vector<fa2_split_item> cand;
      const int cs = make_schedule(ranges, (int)c, &cand);
      if (cs == 0) continue;
      const double cost = schedule_cost(cand, cs, bh, num_units);
      if (cost < best) {
        best = cost;
        plan.swap(cand);
        slots = cs;
      }
    }
  }
  const long long grid = (long long)plan.size() * bh * 4;
  if (grid > 0x7fffffffLL) return FA2_ERR_INVALID_ARG;
  if (items != nullptr) {
    if ((size_t)max_items < plan.size()) return FA2_ERR_INVALID_ARG;
    std::copy(plan.begin(), plan.end(), items);
  }
  *n_items = (int)plan.size();
  *n_slots = slots;
  *workspace_bytes = split_workspace_bytes(B, H, d, slots);
  return FA2_OK;
}

int fa2_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
                  int N, int d, int window_left, int window_right, float scale, void* stream, int in_dtype,
                  int o_dtype, const fa2_split_item* items, int n_items, int n_slots, void* workspace,
                  size_t workspace_bytes) {
  fa2::FwdArgs a;
  const int st = prepare_fwd(q, k, v, o, lse, B, H, H_kv, N, d, window_left, window_right, scale, stream,
                             in_dtype, o_dtype, &a);
  if (st != FA2_OK) return st;
  if (in_dtype != FA2_BF16) return FA2_ERR_UNSUPPORTED;
  const long long T = (N + (long long)fa2::kBf16BlockRows - 1) / fa2::kBf16BlockRows;
  const long long nk = (N + (long long)fa2::kBf16BlockCols - 1) / fa2::kBf16BlockCols;
  if (items == nullptr || !aligned(items, 4) || n_items < 1 || n_items > T * nk) return FA2_ERR_INVALID_ARG;
  if (n_slots < 0 || n_slots > n_items) return FA2_ERR_INVALID_ARG;
  if ((long long)n_items * B * H * 4 > 0x7fffffffLL) return FA2_ERR_INVALID_ARG;
  const size_t need = split_workspace_bytes(B, H, d, n_slots);
  if (n_slots > 0 && (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < need))
    return FA2_ERR_INVALID_ARG;
  // the schedule and the workspace must not overlap each other or any tensor
  const size_t items_bytes = (size_t)n_items * sizeof(fa2_split_item);
  const size_t esz = 2;
  const size_t q_bytes = (size_t)B * H * N * d * esz;
  const size_t kv_bytes = (size_t)B * H_kv * N * d * esz;
  const size_t o_bytes = (size_t)B * H * N * d * (o_dtype == FA2_BF16 ? 2 : 4);
  const size_t lse_bytes = (size_t)B * H * N * sizeof(float);
  const void* bufs[5] = {q, k, v, o, lse};
  const size_t sizes[5] = {q_bytes, kv_bytes, kv_bytes, o_bytes, lse_bytes};
  for (int i = 0; i < 5; ++i) {
    if (i >= 3 && overlaps(items, items_bytes, bufs[i], sizes[i])) return FA2_ERR_INVALID_ARG;
    if (n_slots > 0 && overlaps(workspace, need, bufs[i], sizes[i])) return FA2_ERR_INVALID_ARG;
  }
  if (n_slots > 0 && overlaps(workspace, need, items, items_bytes)) return FA2_ERR_INVALID_ARG;

  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA2_ERR_NO_DEVICE;
  a.items = items;
  a.n_items = n_items;
  a.part = n_slots > 0 ? workspace : nullptr;
  a.n_slots = n_slots;
  hipError_t e = fa2::launch_fwd_bf16(a);
  if (e == hipSuccess) e = fa2::launch_split_merge(a);
  return e == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

int fa2_sparse_plan(int N, int block_q, int block_k, int n_layouts, const unsigned char* block_mask, int causal,
                    int* tile_ptr, unsigned* entries, int max_entries, int* n_entries) {
  if (!block_mask || !n_entries || N < 1 || n_layouts < 1 || max_entries < 0) return FA2_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARG;
  const int br = fa2::kBf16BlockRows, bc = fa2::kBf16BlockCols, slices = fa2::kBf16Waves;
  const int rows_per_slice = br / slices;  // 32
  // every wavefront's rows lie in one query block, every key tile in one key block
  if (block_q < rows_per_slice || block_q % rows_per_slice != 0) return FA2_ERR_UNSUPPORTED;
  if (block_k < bc || block_k % bc != 0) return FA2_ERR_UNSUPPORTED;
  const long long T = (N + (long long)br - 1) / br;
  const long long nk = (N + (long long)bc - 1) / bc;
  const long long nqb = (N + (long long)block_q - 1) / block_q;
  const long long nkb = (N + (long long)block_k - 1) / block_k;
  if (nk >= (1LL << 24) || (long double)n_layouts * T * nk > 2147483647.0L) return FA2_ERR_INVALID_ARG;
  long long count = 0;
  for (long long L = 0; L < n_layouts; ++L) {
    const unsigned char* m = block_mask + L * nqb * nkb;
    for (long long t = 0; t < T; ++t) {
      if (tile_ptr && entries) tile_ptr[L * T + t] = (int)count;
      for (long long j = 0; j < nk; ++j) {
        unsigned bits = 0;
        for (int sl = 0; sl < slices; ++sl) {
          const long long r0 = t * br + (long long)sl * rows_per_slice;
          if (r0 >= N) break;
          const long long r_last = std::min<long long>(r0 + rows_per_slice, N) - 1;
          if (causal && j * bc > r_last) continue;  // the slice's rows see no key of the tile
          if (m[(r0 / block_q) * nkb + (j * bc) / block_k]) bits |= 1u << sl;
        }
        if (bits == 0) continue;
        if (entries) {
          if (count >= max_entries) return FA2_ERR_INVALID_ARG;
          entries[count] = (unsigned)j | (bits << 24);
        }
        ++count;
      }
    }
  }
  if (tile_ptr && entries) tile_ptr[n_layouts * T] = (int)count;
  *n_entries = (int)count;
  return FA2_OK;
}

int fa2_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N,
                   int d, int causal, float scale, void* stream, int in_dtype, int o_dtype, int n_layouts,
                   const int* tile_ptr, const unsigned* entries, int n_entries) {
  if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARG;
  fa2::FwdArgs a;
  const int st = prepare_fwd(q, k, v, o, lse, B, H, H_kv, N, d, -1, causal ? 0 : -1, scale, stream, in_dtype,
                             o_dtype, &a);
  if (st != FA2_OK) return st;
  if (in_dtype != FA2_BF16) return FA2_ERR_UNSUPPORTED;
  if (!(n_layouts == 1 || n_layouts == H || (long long)n_layouts == (long long)B * H)) return FA2_ERR_INVALID_ARG;
  if (!tile_ptr || !aligned(tile_ptr, 4) || n_entries < 0) return FA2_ERR_INVALID_ARG;
  if (n_entries > 0 && (!entries || !aligned(entries, 4))) return FA2_ERR_INVALID_ARG;
  const long long T = (N + (long long)fa2::kBf16BlockRows - 1) / fa2::kBf16BlockRows;
  const size_t ptr_bytes = ((size_t)n_layouts * T + 1) * sizeof(int);
  const size_t ent_bytes = (size_t)n_entries * sizeof(unsigned);
  const size_t o_bytes = (size_t)B * H * N * d * (o_dtype == FA2_BF16 ? 2 : 4);
  const size_t lse_bytes = (size_t)B * H * N * sizeof(float);
  if (overlaps(tile_ptr, ptr_bytes, o, o_bytes) || overlaps(tile_ptr, ptr_bytes, lse, lse_bytes))
    return FA2_ERR_INVALID_ARG;
  if (n_entries > 0 && (overlaps(entries, ent_bytes, o, o_bytes) || overlaps(entries, ent_bytes, lse, lse_bytes)))
    return FA2_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA2_ERR_NO_DEVICE;
  a.sp_ptr = tile_ptr;
  // with no entries the kernel never reads the entry array; any valid
  // pointer will do
  a.sp_ent = n_entries > 0 ? entries : reinterpret_cast<const unsigned*>(tile_ptr);
  a.n_layouts = n_layouts;
  a.n_entries = n_entries;
  const hipError_t e = fa2::launch_fwd_bf16(a);
  return e == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

int fa2_decode_paged_workspace(int B, int H, int H_kv, int n_q, int d, int max_context, int split_keys,
                               int num_units, int* split_keys_out, size_t* workspace_bytes) {
  if (!split_keys_out || !workspace_bytes) return FA2_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || H_kv < 1 || H % H_kv != 0 || n_q < 1 || max_context < 1) return FA2_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA2_ERR_UNSUPPORTED;
  if ((long long)(H / H_kv) * n_q > fa2::kBf16BlockRows) return FA2_ERR_UNSUPPORTED;
  const int bc = fa2::kBf16BlockCols;
  if (split_keys < 0 || split_keys % bc != 0) return FA2_ERR_INVALID_ARG;
  if (split_keys == 0) {
    // At least four key tiles per chunk unless the context is shorter, and:
    // - groups of up to 128 query rows run one wavefront per (chunk, group,
    //   block of 32 rows), four per compute unit: enough chunks at the
    //   longest context for one chunk per wavefront slot (more chunks start
    //   a second, partial round; fewer leave slots idle), or four per
    //   sequence once the wavefronts of one chunk alone fill the slots
    //   (smaller chunks balance the rounds);
    // - larger groups run workgroups of the forward kernel: about eight per
    //   compute unit at the longest context (about four on average for a
    //   mixed batch).
    if (num_units < 1) return FA2_ERR_INVALID_ARG;
    const long long groups = (long long)B * H_kv;
    const long long rows = (long long)(H / H_kv) * n_q;
    const long long slots = rows <= 128 ? 4LL * num_units : 0;
    const long long waves = groups * ((rows + 31) / 32);  // per chunk
    const long long want = slots > 0 ? (waves < slots ? (slots + waves - 1) / waves : 4)
                                     : std::max<long long>(1, (8LL * num_units + groups - 1) / groups);
    long long keys = (max_context + want - 1) / want;
    keys = (keys + bc - 1) / bc * bc;
    const long long floor_keys = std::min<long long>(4 * bc, ((long long)max_context + bc - 1) / bc * bc);
    split_keys = (int)std::max(keys, floor_keys);
  }
  const long long chunks = ((long long)max_context + split_keys - 1) / split_keys;
  const long double bytes = (long double)B * H_kv * chunks * (H / H_kv) * n_q * ((long double)d * 4 + 8);
  if (bytes > (long double)(1LL << 50) || (long double)chunks * B * H_kv > 2147483647.0L) return FA2_ERR_INVALID_ARG;
  *split_keys_out = split_keys;
  *workspace_bytes = (size_t)bytes;
  return FA2_OK;
}

namespace {

// fa2_decode_paged and fa2_decode_paged_noalloc: with from_scratch the
// partials go to the static per-device scratch instead of `workspace`.
int decode_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int H,
                 int H_kv, int n_q, int d, float scale, const int* page_table, int max_pages,
                 const int* context_lens, int max_context, int page_size, int n_pages, int split_keys,
                 void* workspace, size_t workspace_bytes, void* stream, int in_dtype, int o_dtype,
                 bool from_scratch) {
  if (!q || !k_cache || !v_cache || !o || !lse || !page_table || !context_lens) return FA2_ERR_INVALID_ARG;
  if (!from_scratch && !workspace) return FA2_ERR_INVALID_ARG;
  if (!is_dtype(in_dtype) || !is_dtype(o_dtype)) return FA2_ERR_INVALID_ARG;
  if (max_pages < 1 || n_pages < 1 || page_size < 1 || split_keys < 1) return FA2_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || scale < 0.f) return FA2_ERR_INVALID_ARG;
  int split_out = 0;
  size_t need = 0;
  const int st = fa2_decode_paged_workspace(B, H, H_kv, n_q, d, max_context, split_keys, 0, &split_out, &need);
  if (st != FA2_OK) return st;
  if (in_dtype != FA2_BF16) return FA2_ERR_UNSUPPORTED;
  const int bc = fa2::kBf16BlockCols;
  if (page_size % bc != 0) return FA2_ERR_UNSUPPORTED;  // a key tile must lie in one page
  if ((long double)n_pages * page_size * H_kv * d > (long double)(1LL << 60)) return FA2_ERR_INVALID_ARG;
  if ((long double)max_pages * page_size > 2147483647.0L) return FA2_ERR_INVALID_ARG;
  if (from_scratch) {
    if (need > FA2_DECODE_SCRATCH_BYTES) return FA2_ERR_SCRATCH;
  } else if (workspace_bytes < need) {
    return FA2_ERR_INVALID_ARG;
  }
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      (!from_scratch && !aligned(workspace, 16)) || !aligned(page_table, 4) || !aligned(context_lens, 4))
    return FA2_ERR_INVALID_ARG;
  const size_t rows = (size_t)B * H * n_q;
  const size_t q_bytes = rows * d * 2;
  const size_t o_bytes = rows * d * (o_dtype == FA2_BF16 ? 2 : 4);
  const size_t lse_bytes = rows * sizeof(float);
  const size_t cache_bytes = (size_t)n_pages * page_size * H_kv * d * 2;
  const size_t table_bytes = (size_t)B * max_pages * sizeof(int);
  const size_t lens_bytes = (size_t)B * sizeof(int);
  // written buffers against everything else (the static scratch is its own
  // allocation and cannot overlap a caller's buffer)
  const int n_out = from_scratch ? 2 : 3;
  const void* outs[3] = {o, lse, workspace};
  const size_t out_sz[3] = {o_bytes, lse_bytes, need};
  const void* ins[6] = {q, k_cache, v_cache, page_table, context_lens, nullptr};
  const size_t in_sz[6] = {q_bytes, cache_bytes, cache_bytes, table_bytes, lens_bytes, 0};
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < 5; ++j)
      if (overlaps(outs[i], out_sz[i], ins[j], in_sz[j])) return FA2_ERR_INVALID_ARG;
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(outs[i], out_sz[i], outs[j], out_sz[j])) return FA2_ERR_INVALID_ARG;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA2_ERR_NO_DEVICE;
  if (from_scratch && fa2::decode_scratch(&workspace) != hipSuccess) return FA2_ERR_LAUNCH;

  fa2::FwdArgs a;
  a.q = q; a.k = k_cache; a.v = v_cache; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.Hkv = H_kv; a.N = max_context; a.d = d;
  a.causal = true;
  a.wl = -1;
  a.wr = 0;
  a.scale = scale;
  a.o_bf16 = (o_dtype == FA2_BF16);
  const char* dbg = std::getenv("FA2_DEBUG_POISON");
  a.poison = dbg != nullptr && dbg[0] != '\0' && dbg[0] != '0';
  a.part = workspace;
  a.n_slots = (int)(((long long)max_context + split_keys - 1) / split_keys);
  a.paged.page_table = page_table;
  a.paged.ctx_lens = context_lens;
  a.paged.max_pages = max_pages;
  a.paged.page_size = page_size;
  a.paged.n_pages = n_pages;
  a.paged.n_q = n_q;
  a.paged.chunk_tiles = split_keys / bc;
  a.paged.kv_heads = H_kv;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = fa2::launch_decode_paged(a);
  return e == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

}  // namespace

int fa2_decode_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int H,
                     int H_kv, int n_q, int d, float scale, const int* page_table, int max_pages,
                     const int* context_lens, int max_context, int page_size, int n_pages, int split_keys,
                     void* workspace, size_t workspace_bytes, void* stream, int in_dtype, int o_dtype) {
  return decode_paged(q, k_cache, v_cache, o, lse, B, H, H_kv, n_q, d, scale, page_table, max_pages, context_lens,
                      max_context, page_size, n_pages, split_keys, workspace, workspace_bytes, stream, in_dtype,
                      o_dtype, false);
}

int fa2_decode_paged_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B,
                             int H, int H_kv, int n_q, int d, float scale, const int* page_table, int max_pages,
                             const int* context_lens, int max_context, int page_size, int n_pages, int split_keys,
                             void* stream, int in_dtype, int o_dtype) {
  return decode_paged(q, k_cache, v_cache, o, lse, B, H, H_kv, n_q, d, scale, page_table, max_pages, context_lens,
                      max_context, page_size, n_pages, split_keys, nullptr, 0, stream, in_dtype, o_dtype, true);
}

int fa2_fp8_pack_workspace(int B, int H, int N, size_t* workspace_bytes) {
  if (!workspace_bytes || B < 1 || H < 1 || N < 1) return FA2_ERR_INVALID_ARG;
  if ((long double)B * H * N > (long double)(1LL << 40)) return FA2_ERR_INVALID_ARG;
  *workspace_bytes = (size_t)B * H * fa2::fp8_pack_chunks(N) * sizeof(float);
  return FA2_OK;
}

int fa2_fp8_pack(const void* x, int B, int H, int N, int d, const float* signs, void* codes, float* scales,
                 void* workspace, size_t workspace_bytes, void* stream) {
  if (!x || !codes || !scales || !workspace) return FA2_ERR_INVALID_ARG;
  size_t need = 0;
  if (fa2_fp8_pack_workspace(B, H, N, &need) != FA2_OK) return FA2_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA2_ERR_UNSUPPORTED;
  if (workspace_bytes < need) return FA2_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(workspace, 4))
    return FA2_ERR_INVALID_ARG;
  fa2::Fp8Signs sg = {{0u, 0u, 0u, 0u}};
  if (signs) {
    for (int i = 0; i < d; ++i) {
      if (signs[i] == -1.0f) sg.bits[i >> 5] |= 1u << (i & 31);
      else if (signs[i] != 1.0f) return FA2_ERR_INVALID_ARG;
    }
  }
  const size_t x_bytes = (size_t)B * H * N * d * 2, c_bytes = (size_t)B * H * N * d;
  const size_t s_bytes = (size_t)B * H * sizeof(float);
  const void* bufs[4] = {x, codes, scales, workspace};
  const size_t sz[4] = {x_bytes, c_bytes, s_bytes, need};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(bufs[i], sz[i], bufs[j], sz[j])) return FA2_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA2_ERR_NO_DEVICE;
  fa2::Fp8PackArgs a;
  a.x = x; a.BH = B * H; a.N = N; a.d = d;
  a.rotate = signs != nullptr;
  a.signs = sg;
  a.codes = codes; a.scales = scales; a.partial = static_cast<float*>(workspace);
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return fa2::launch_fp8_pack(a) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

int fa2_fwd_fp8(const void* q8, const float* q_scale, const void* k8, const float* k_scale, const void* v,
                void* o, float* lse, int B, int H, int H_kv, int N, int d, int causal, float scale, void* stream,
                int o_dtype) {
  if (!q8 || !q_scale || !k8 || !k_scale || !v || !o || !lse) return FA2_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARG;
  if (H_kv < 1 || H < 1 || H % H_kv != 0 || !is_dtype(o_dtype)) return FA2_ERR_INVALID_ARG;
  const int st = check_sizes(B, H, N, d, FA2_BF16);
  if (st != FA2_OK) return st;
  if (!std::isfinite(scale) || scale < 0.f) return FA2_ERR_INVALID_ARG;
  if (!aligned(q8, 16) || !aligned(k8, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(q_scale, 4) || !aligned(k_scale, 4))
    return FA2_ERR_INVALID_ARG;
  const size_t rows = (size_t)B * H * N, kv_rows = (size_t)B * H_kv * N;
  const void* ins[5] = {q8, k8, v, q_scale, k_scale};
  const size_t in_sz[5] = {rows * d, kv_rows * d, kv_rows * d * 2, (size_t)B * H * 4, (size_t)B * H_kv * 4};
  const size_t o_bytes = rows * d * (o_dtype == FA2_BF16 ? 2 : 4), lse_bytes = rows * 4;
  for (int i = 0; i < 5; ++i)
    if (overlaps(o, o_bytes, ins[i], in_sz[i]) || overlaps(lse, lse_bytes, ins[i], in_sz[i])) return FA2_ERR_INVALID_ARG;
  if (overlaps(o, o_bytes, lse, lse_bytes)) return FA2_ERR_INVALID_ARG;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA2_ERR_NO_DEVICE;
  fa2::FwdArgs a;
  a.q = q8; a.k = k8; a.v = v; a.o = o; a.lse = lse;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.Hkv = H_kv;
  a.causal = causal != 0;
  a.wl = -1;
  a.wr = causal ? 0 : -1;
  a.scale = scale;
  a.o_bf16 = (o_dtype == FA2_BF16);
  a.poison = false;
  a.fp8 = true;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return fa2::launch_fwd_bf16(a) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
            const float* lse, float* delta, void* dq, void* dk, void* dv, int B, int H, int N, int d,
            int causal, float scale, void* stream, int in_dtype, int o_dtype, int grad_dtype) {
  return fa2_bwd_gqa(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H, N, d, causal, scale, stream,
                     in_dtype, o_dtype, grad_dtype);
}

int fa2_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, float* delta, void* dq, void* dk, void* dv, int B, int H, int H_kv,
                int N, int d, int causal, float scale, void* stream, int in_dtype, int o_dtype,
                int grad_dtype) {
  if (causal != 0 && causal != 1) return FA2_ERR_INVALID_ARG;
  return fa2_bwd_window(q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, H_kv, N, d, -1, causal ? 0 : -1,
                        scale, stream, in_dtype, o_dtype, grad_dtype);
}

int fa2_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, float* delta, void* dq, void* dk, void* dv, int B, int H, int H_kv,
                   int N, int d, int window_left, int window_right, float scale, void* stream,
                   int in_dtype, int o_dtype, int grad_dtype) {
  if (!q || !k || !v || !o || !dout || !lse || !delta || !dq || !dk || !dv) return FA2_ERR_INVALID_ARG;
  if (H_kv < 1 || H < 1 || H % H_kv != 0) return FA2_ERR_INVALID_ARG;
  if (window_left < -1 || window_right < -1) return FA2_ERR_INVALID_ARG;
  if (!is_dtype(o_dtype) || !is_dtype(grad_dtype)) return FA2_ERR_INVALID_ARG;
  const int st = check_sizes(B, H, N, d, in_dtype);
  if (st != FA2_OK) return st;
  if (!std::isfinite(scale) || scale < 0.f) return FA2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(delta, 4))
    return FA2_ERR_INVALID_ARG;
  const size_t elems = (size_t)B * H * N * d;
  const size_t kv_elems = (size_t)B * H_kv * N * d;
  const size_t esz = in_dtype == FA2_BF16 ? 2 : 4;
  const size_t gsz = grad_dtype == FA2_BF16 ? 2 : 4;
  const size_t o_bytes = elems * (o_dtype == FA2_BF16 ? 2 : 4);
  const size_t row_bytes = (size_t)B * H * N * sizeof(float);
  const void* ins[6] = {q, k, v, dout, o, lse};
  const size_t in_sz[6] = {elems * esz, kv_elems * esz, kv_elems * esz, elems * esz, o_bytes, row_bytes};
  const void* outs[4] = {dq, dk, dv, delta};
  const size_t out_sz[4] = {elems * gsz, kv_elems * gsz, kv_elems * gsz, row_bytes};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_sz[i], ins[j], in_sz[j])) return FA2_ERR_INVALID_ARG;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_sz[i], outs[j], out_sz[j])) return FA2_ERR_INVALID_ARG;
  }
  if (in_dtype != FA2_BF16 || (d != 64 && d != 128)) return FA2_ERR_UNSUPPORTED;

  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA2_ERR_NO_DEVICE;

  fa2::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse; a.delta = delta;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.B = B; a.H = H; a.N = N; a.d = d;
  a.Hkv = H_kv;
  // a bound of N or more keys is no bound
  a.wl = window_left >= N ? -1 : window_left;
  a.wr = window_right >= N ? -1 : window_right;
  a.causal = (a.wl == -1 && a.wr == 0);
  a.scale = scale;
  a.o_bf16 = (o_dtype == FA2_BF16);
  a.grad_bf16 = (grad_dtype == FA2_BF16);
  a.stream = reinterpret_cast<hipStream_t>(stream);
  return fa2::launch_bwd_bf16(a) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

}  // extern "C"
