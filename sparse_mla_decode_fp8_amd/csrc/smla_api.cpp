// C ABI of libsmla.so (declared in include/smla.h): argument validation,
// work planning (split factor, workspace layout) and kernel launches on the
// caller's stream.  No allocation and no host synchronisation on the forward
// path.

#include <hip/hip_runtime.h>
#include <limits.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "smla.h"
#include "smla_internal.h"

namespace {

// The last failing call's message (a fixed buffer: reporting an error
// allocates nothing).
thread_local char g_err[512];

void clear_err() { g_err[0] = 0; }

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(SMLA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Process-wide tuning knobs (sparse_mla_set_option; benchmarks and tests).
// Atomic, so concurrent forwards read a consistent value; a forward reads
// each once, so a change applies to the forwards that start after it.
std::atomic<int64_t> g_split_override{0};  // 0 = automatic
std::atomic<int64_t> g_plan_override{0};   // 0 = automatic, 1 = never plan, 2 = always plan
std::atomic<int64_t> g_persist_override{0};  // 0 = automatic, 1 = one unit per block always

// Index reads use 32-bit byte offsets; the kernels read up to a few tiles past
// a row's end, so leave headroom below 2^32 bytes.
constexpr int64_t kMaxNnz = (int64_t(1) << 30) - 4096;

// Device address of the zero record, per device (looked up once per device).
std::mutex g_zero_mu;
const uint8_t* g_zero_ptr[64] = {};

// The device a stream belongs to (the current device for the null stream):
// the kernels run there, so per-device addresses are that device's.
hipError_t stream_device(hipStream_t s, int* dev) {
  if (!s) return hipGetDevice(dev);
  hipDevice_t d = 0;
  const hipError_t e = hipStreamGetDevice(s, &d);
  if (e == hipSuccess) *dev = (int)d;
  return e;
}

// The zero record's address on device dev (the symbol is looked up with dev
// current, once per device; the calling thread's current device is restored).
hipError_t zero_record(int dev, const uint8_t** out) {
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_zero_mu);
  if (!g_zero_ptr[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = smla::zero_record_address(&g_zero_ptr[dev]);
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) {
      g_zero_ptr[dev] = nullptr;
      return e;
    }
  }
  *out = g_zero_ptr[dev];
  return hipSuccess;
}

// Compute units of the current device (queried once per device).
std::atomic<int> g_cus[64];

// Head counts the forward implements (the QK and V dims are fixed by the record).
bool heads_ok(int32_t H) { return H >= 1 && H <= SMLA_MAX_HEADS; }

int device_cus(int dev = -1) {
  int cus = 0;
  if (dev < 0 && hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && (cus = g_cus[dev].load(std::memory_order_relaxed)) > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  if (dev >= 0 && dev < 64) g_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// Chunks per row.  Rows are independent, so split only when there are too few
// rows to give every CU a unit; never split below one tile per chunk.  With
// padded slices (has_invalid) the rows' real lengths differ, and a batch of
// about one row per CU is bounded by its longest rows: two chunks per row,
// queued longest first, let those rows use two CUs.
// `dev`: the device the forward runs on (-1: the current device).
int choose_split(int32_t T, int32_t H, int64_t nnz, bool has_invalid, int dev) {
  const int64_t forced = g_split_override.load(std::memory_order_relaxed);
  if (forced > 0) return (int)forced;
  if (T <= 0) return 1;
  const int tile = smla::tile_tokens(H);
  const int64_t avg_tiles = (nnz / T + tile - 1) / tile;
  const int cus = device_cus(dev);
  const int64_t units = (int64_t)T * smla::head_groups(H);  // unsplit units
  if (units >= cus) return (has_invalid && 2 * units <= 3 * (int64_t)cus && avg_tiles >= 2) ? 2 : 1;
  int64_t s = (cus + units - 1) / units;
  if (s > avg_tiles) s = avg_tiles;
  if (s > SMLA_MAX_SPLIT) s = SMLA_MAX_SPLIT;
  return s < 1 ? 1 : (int)s;
}

struct Layout {
  int S;
  size_t row_tiles, order, desc, part_lse, part_o, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// `partials`: the V4.1 path writes chunk partials for every row (its
// epilogue runs in the combine), whatever the split.  The size is that of
// the larger split (a padded batch's), so one workspace serves both.
Layout layout(int32_t T, int32_t H, int64_t nnz, bool partials, bool has_invalid, int dev) {
  Layout L{};
  const int s_max = choose_split(T, H, nnz, true, dev);
  L.S = choose_split(T, H, nnz, has_invalid, dev);
  size_t off = 0;
  L.row_tiles = off;
  off = align256(off + sizeof(int32_t) * (size_t)T);
  L.order = off;
  off = align256(off + sizeof(int32_t) * (size_t)T);
  L.desc = off;
  off = align256(off + 4 * sizeof(int32_t) * (size_t)T);
  L.part_lse = off;
  L.part_o = off;
  if (s_max > 1 || partials) {
    off = align256(off + sizeof(float) * (size_t)T * s_max * H);
    L.part_o = off;
    off = align256(off + sizeof(uint16_t) * (size_t)T * s_max * H * 512);  // f16 partial outputs
  }
  L.total = off;
  return L;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// ---- kernel timing (benchmarks)
struct Prof {
  std::mutex mu;
  bool active = false;
  int cap = 0;
  int used = 0;  // event pairs used
  std::vector<hipEvent_t> ev;  // 2 per pair
  std::vector<int> kind;       // per pair
} g_prof;

// Runs `launch(ev)`; while profiling, ev carries an event pair that the
// launch attaches to its kernel dispatches (hipExtLaunchKernel), so the pair
// brackets the kernels' execution and not the queueing around them.
template <class F>
hipError_t timed(int kind, F&& launch) {
  smla::Events ev;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.active && g_prof.used < g_prof.cap) {
      const int slot = g_prof.used++;
      g_prof.kind[slot] = kind;
      ev.start = g_prof.ev[2 * slot];
      ev.stop = g_prof.ev[2 * slot + 1];
    }
  }
  return launch(ev);
}

}  // namespace

extern "C" {

int sparse_mla_supported(int32_t num_heads, int32_t head_dim_qk, int32_t dv) {
  return heads_ok(num_heads) && head_dim_qk == 576 && dv == 512;
}

int64_t sparse_mla_workspace_bytes(int32_t T, int32_t H, int64_t nnz) {
  if (T < 0 || nnz < 0) return fail(SMLA_EINVAL, "T and nnz must be >= 0 (T=%d nnz=%lld)", T, (long long)nnz);
  if (!heads_ok(H)) return fail(SMLA_EUNSUPPORTED, "num_heads must be in [1, %d], got %d", SMLA_MAX_HEADS, H);
  return (int64_t)layout(T, H, nnz, false, true, -1).total;
}

int32_t sparse_mla_split_for(int32_t T, int32_t H, int64_t nnz, int32_t has_invalid) {
  if (T < 0 || nnz < 0) return fail(SMLA_EINVAL, "T and nnz must be >= 0 (T=%d nnz=%lld)", T, (long long)nnz);
  if (!heads_ok(H)) return fail(SMLA_EUNSUPPORTED, "num_heads must be in [1, %d], got %d", SMLA_MAX_HEADS, H);
  return choose_split(T, H, nnz, has_invalid != 0, -1);
}

}  // extern "C"

namespace {

// Where the keys live: one contiguous cache, or two paged pools.
struct KeySource {
  smla::KeyMode km;
  const uint8_t* kv;
  const uint8_t* pool[2];
  int64_t pool_stride[2];
  int32_t pool_shift[2];
};

// Pool descriptors of the paged entry points: a key's bytes in a page are
// `key_bytes` (656 for fp8_ds_mla records, 576 + 8 for V4.1 keys).
int parse_pools(const smla_kv_pool* pools, int64_t key_bytes, KeySource& ks) {
  if (!pools) return fail(SMLA_EINVAL, "pools is null (two pool descriptors are required)");
  ks.km.paged = 1;
  for (int i = 0; i < 2; ++i) {
    const smla_kv_pool& pl = pools[i];
    if (!pl.base) {  // absent: its entries are not keys
      ks.km.present[i] = 0;
      continue;
    }
    const int64_t pr = pl.page_records;
    if (pr < 1 || pr > (int64_t(1) << 30) || (pr & (pr - 1)) != 0)
      return fail(SMLA_EINVAL, "pool %d: page_records must be a power of two in [1, 2^30], got %lld", i, (long long)pr);
    if (!aligned(pl.base, 16)) return fail(SMLA_EINVAL, "pool %d: base must be 16-byte aligned", i);
    if (pl.page_stride % 16 != 0 || pl.page_stride < pr * key_bytes)
      return fail(SMLA_EINVAL, "pool %d: page_stride must be a multiple of 16 and >= page_records * %lld bytes, got %lld",
                  i, (long long)key_bytes, (long long)pl.page_stride);
    if (pl.page_stride > INT64_MAX / (int64_t(1) << 31))
      return fail(SMLA_EINVAL, "pool %d: page_stride too large: %lld", i, (long long)pl.page_stride);
    ks.km.present[i] = 1;
    ks.pool[i] = (const uint8_t*)pl.base;
    ks.pool_stride[i] = pl.page_stride;
    int sh = 0;
    while ((int64_t(1) << sh) < pr) ++sh;
    ks.pool_shift[i] = sh;
  }
  return SMLA_OK;
}

// The V4.1 key record's outputs (the combine's epilogue).
struct V41Out {
  const int32_t* pos;
  const float* cos_sin;
  int32_t n_pos;
  uint8_t* xo;
  uint8_t* xos;
  float* y_out;
};

// The forward shared by the entry points (keys already validated).  With
// `v41`, the keys are V4.1 records (out unused; the combine writes xo, xos).
int fwd_impl(const void* q, int64_t q_stride_t, int64_t q_stride_h, const KeySource& ks,
             const int32_t* indptr, const int32_t* indices, int64_t nnz,
             int32_t T, int32_t H, float sm_scale, int32_t has_invalid, const float* sink,
             void* out, int64_t o_stride_t, int64_t o_stride_h, float* lse,
             void* workspace, int64_t workspace_bytes, void* stream, const V41Out* v41 = nullptr,
             bool noalloc = false) {
  if (!heads_ok(H)) return fail(SMLA_EUNSUPPORTED, "num_heads must be in [1, %d], got %d", SMLA_MAX_HEADS, H);
  if (v41 && H > 16) return fail(SMLA_EUNSUPPORTED, "the V4.1 record path implements 1 to 16 heads, got %d", H);
  if (T < 0) return fail(SMLA_EINVAL, "T must be >= 0, got %d", T);
  if (nnz < 0) return fail(SMLA_EINVAL, "nnz must be >= 0, got %lld", (long long)nnz);
  if (nnz > kMaxNnz) return fail(SMLA_EINVAL, "nnz must be <= %lld (32-bit bounded index reads), got %lld", (long long)kMaxNnz, (long long)nnz);
  if (!isfinite(sm_scale)) return fail(SMLA_EINVAL, "sm_scale must be finite");
  if (T == 0) return SMLA_OK;
  if (!q || !indptr || !(out || v41) || !(workspace || noalloc))
    return fail(SMLA_EINVAL, "null pointer (q, indptr, out and workspace are required)");
  if (nnz > 0 && !indices) return fail(SMLA_EINVAL, "indices is null but nnz > 0");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(SMLA_EINVAL, "q and out must be 16-byte aligned");
  if (lse && !aligned(lse, 4)) return fail(SMLA_EINVAL, "lse must be 4-byte aligned");
  if (sink && !aligned(sink, 4)) return fail(SMLA_EINVAL, "sink must be 4-byte aligned");
  if (!aligned(workspace, 256)) return fail(SMLA_EINVAL, "workspace must be 256-byte aligned");
  if (q_stride_t < 0 || q_stride_h < 0 || o_stride_t < 0 || o_stride_h < 0 ||
      (q_stride_t | q_stride_h | o_stride_t | o_stride_h) % 8 != 0)
    return fail(SMLA_EINVAL, "strides must be non-negative multiples of 8 elements");
  // the split and the workspace layout are those of the stream's device
  // (a failed device lookup is reported after the argument checks)
  hipStream_t s = (hipStream_t)stream;
  int dev = -1;
  hipError_t ez = stream_device(s, &dev);
  const Layout L = layout(T, H, nnz, v41 != nullptr, has_invalid != 0, ez == hipSuccess ? dev : -1);
  // every grid of the call (forward units; the combine's one block per row
  // and head) must fit a 32-bit launch dimension
  if (8 * (((int64_t)T + 7) / 8) * std::max<int64_t>((int64_t)L.S * smla::head_groups(H), H) > INT32_MAX)
    return fail(SMLA_EINVAL, "T = %d rows need more blocks than one launch holds", T);
  if (noalloc && (int64_t)L.total > SMLA_NOALLOC_SCRATCH_BYTES)
    return fail(SMLA_EWORKSPACE, "this forward needs %lld bytes of scratch; the static scratch holds %lld "
                "(call sparse_mla_fwd with a workspace)", (long long)L.total, (long long)SMLA_NOALLOC_SCRATCH_BYTES);
  if (!noalloc && workspace_bytes < (int64_t)L.total)
    return fail(SMLA_EWORKSPACE, "workspace has %lld bytes, needs %lld", (long long)workspace_bytes, (long long)L.total);

  if (ez != hipSuccess) return hip_fail(ez, "stream device");
  const uint8_t* zero = nullptr;
  ez = zero_record(dev, &zero);
  if (ez != hipSuccess) return hip_fail(ez, "zero record lookup");
  if (noalloc) {  // the device's static scratch stands in for the workspace
    ez = smla::noalloc_scratch(dev, &workspace);
    if (ez != hipSuccess) return hip_fail(ez, "static scratch lookup");
  }
  uint8_t* ws = (uint8_t*)workspace;
  int32_t* row_tiles = (int32_t*)(ws + L.row_tiles);
  int32_t* order = (int32_t*)(ws + L.order);
  int32_t* desc = (int32_t*)(ws + L.desc);
  const uint32_t idx_bytes = (uint32_t)(nnz * 4);

  // Longest-first order only pays when there are more units than CUs (one
  // forward block fits a CU): otherwise every unit starts at once and the
  // order cannot shorten the slowest.  Without an order there is nothing to
  // plan: each forward block takes its row's length from indptr and, with
  // has_invalid, trims the trailing masked entries by a scan of its own row.
  const int64_t plan_opt = g_plan_override.load(std::memory_order_relaxed);
  const bool sort = plan_opt == 1   ? false
                    : plan_opt == 2 ? true
                                    : (int64_t)T * L.S * smla::head_groups(H) > device_cus(dev);
  hipError_t e = hipSuccess;
  if (sort) {
    smla::PlanParams pp{indptr, indices, idx_bytes, T, smla::tile_tokens(H), has_invalid ? 1 : 0,
                        ks.km, row_tiles, order, desc};
    e = timed(0, [&](smla::Events ev) { return smla::launch_plan(pp, sort, ev, s); });
    if (e != hipSuccess) return hip_fail(e, "plan kernel launch");
  }

  smla::FwdParams fp{};
  fp.q = (const uint16_t*)q;
  fp.q_st = q_stride_t;
  fp.q_sh = q_stride_h;
  fp.kv = ks.kv;
  fp.zero = zero;
  fp.indptr = indptr;
  fp.indices = indices;
  fp.idx_bytes = idx_bytes;
  fp.T = T;
  fp.H = H;
  fp.S = L.S;
  fp.c_log2 = (float)((double)sm_scale * 1.4426950408889634074);
  fp.out = (uint16_t*)out;
  fp.o_st = o_stride_t;
  fp.o_sh = o_stride_h;
  fp.lse = lse;
  fp.row_tiles = sort ? row_tiles : nullptr;
  fp.scan = (!sort && has_invalid) ? 1 : 0;
  // slices laid out at a fixed stride (a [T, top-k] index buffer) let each
  // block start its index reads before indptr arrives
  fp.stride = (!sort && nnz % T == 0 && nnz / T > 0) ? (int32_t)(nnz / T) : 0;
  fp.order = sort ? order : nullptr;
  fp.desc = sort ? desc : nullptr;
  fp.part_o = (uint16_t*)(ws + L.part_o);
  fp.part_lse = (float*)(ws + L.part_lse);
  fp.km = ks.km;
  for (int i = 0; i < 2; ++i) {
    fp.pool[i] = ks.pool[i];
    fp.pool_stride[i] = ks.pool_stride[i];
    fp.pool_shift[i] = ks.pool_shift[i];
  }
  fp.sink = sink;
  fp.hg = smla::head_groups(H);
  // with the plan (more units than CUs), kernels that can run several units
  // per block get a persistent grid of one block per CU
  fp.persist = (sort && g_persist_override.load(std::memory_order_relaxed) == 0) ? (device_cus(dev) / 8) * 8 : 0;
  if (v41) {
    fp.sink = nullptr;  // partials never hold the sink: the combine folds it in
    e = timed(1, [&](smla::Events ev) { return smla::launch_fwd41(fp, ev, s); });
    if (e != hipSuccess) return hip_fail(e, "forward kernel launch");
    smla::Combine41Params cp{T, H, L.S, sink, fp.order, fp.part_o, fp.part_lse,
                             v41->pos, v41->cos_sin, v41->n_pos, v41->xo, v41->xos, lse, v41->y_out};
    e = timed(2, [&](smla::Events ev) { return smla::launch_combine41(cp, ev, s); });
    if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
    return SMLA_OK;
  }
  e = timed(1, [&](smla::Events ev) { return smla::launch_fwd(fp, ev, s); });
  if (e != hipSuccess) return hip_fail(e, "forward kernel launch");

  if (L.S > 1) {
    smla::CombineParams cp{T, H, L.S, sink, fp.order, fp.part_o, fp.part_lse, fp.out, o_stride_t, o_stride_h, lse};
    e = timed(2, [&](smla::Events ev) { return smla::launch_combine(cp, ev, s); });
    if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  }
  return SMLA_OK;
}

}  // namespace

extern "C" {

int sparse_mla_fwd(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                   const void* kv, int64_t n_kv,
                   const int32_t* indptr, const int32_t* indices, int64_t nnz,
                   int32_t T, int32_t H, float sm_scale, int32_t has_invalid,
                   void* out, int64_t o_stride_t, int64_t o_stride_h,
                   float* lse,
                   void* workspace, int64_t workspace_bytes,
                   void* stream) {
  clear_err();
  if (n_kv < 0 || n_kv > INT64_MAX / smla::kRecordBytes) return fail(SMLA_EINVAL, "n_kv out of range: %lld", (long long)n_kv);
  if (T > 0 && !kv) return fail(SMLA_EINVAL, "null pointer (kv is required)");
  if (!aligned(kv, 16)) return fail(SMLA_EINVAL, "kv must be 16-byte aligned");
  KeySource ks{};
  ks.km = smla::KeyMode{0, {1, 1}};
  ks.kv = (const uint8_t*)kv;
  return fwd_impl(q, q_stride_t, q_stride_h, ks, indptr, indices, nnz, T, H, sm_scale, has_invalid, nullptr,
                  out, o_stride_t, o_stride_h, lse, workspace, workspace_bytes, stream);
}

int sparse_mla_fwd_noalloc(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                           const void* kv, int64_t n_kv,
                           const int32_t* indptr, const int32_t* indices, int64_t nnz,
                           int32_t T, int32_t H, float sm_scale, int32_t has_invalid,
                           void* out, int64_t o_stride_t, int64_t o_stride_h,
                           float* lse, void* stream) {
  clear_err();
  if (n_kv < 0 || n_kv > INT64_MAX / smla::kRecordBytes) return fail(SMLA_EINVAL, "n_kv out of range: %lld", (long long)n_kv);
  if (T > 0 && !kv) return fail(SMLA_EINVAL, "null pointer (kv is required)");
  if (!aligned(kv, 16)) return fail(SMLA_EINVAL, "kv must be 16-byte aligned");
  KeySource ks{};
  ks.km = smla::KeyMode{0, {1, 1}};
  ks.kv = (const uint8_t*)kv;
  return fwd_impl(q, q_stride_t, q_stride_h, ks, indptr, indices, nnz, T, H, sm_scale, has_invalid, nullptr,
                  out, o_stride_t, o_stride_h, lse, nullptr, 0, stream, nullptr, /*noalloc=*/true);
}

int sparse_mla_fwd_paged(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                         const smla_kv_pool* pools,
                         const int32_t* indptr, const int32_t* indices, int64_t nnz,
                         int32_t T, int32_t H, float sm_scale, int32_t has_invalid,
                         const float* sink,
                         void* out, int64_t o_stride_t, int64_t o_stride_h,
                         float* lse,
                         void* workspace, int64_t workspace_bytes,
                         void* stream) {
  clear_err();
  KeySource ks{};
  const int rc = parse_pools(pools, smla::kRecordBytes, ks);
  if (rc != SMLA_OK) return rc;
  return fwd_impl(q, q_stride_t, q_stride_h, ks, indptr, indices, nnz, T, H, sm_scale, has_invalid, sink,
                  out, o_stride_t, o_stride_h, lse, workspace, workspace_bytes, stream);
}

int64_t sparse_mla_v41_workspace_bytes(int32_t T, int32_t H, int64_t nnz) {
  if (T < 0 || nnz < 0) return fail(SMLA_EINVAL, "T and nnz must be >= 0 (T=%d nnz=%lld)", T, (long long)nnz);
  if (H < 1 || H > 16) return fail(SMLA_EUNSUPPORTED, "the V4.1 record path implements 1 to 16 heads, got %d", H);
  return (int64_t)layout(T, H, nnz, true, true, -1).total;
}

int sparse_mla_fwd_v41(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                       const smla_kv_pool* pools,
                       const int32_t* indptr, const int32_t* indices, int64_t nnz,
                       int32_t T, int32_t H, float sm_scale, int32_t has_invalid,
                       const float* sink, const int32_t* pos, const float* cos_sin, int32_t n_pos,
                       void* xo, void* xo_scales, float* lse, float* y_out,
                       void* workspace, int64_t workspace_bytes, void* stream) {
  clear_err();
  KeySource ks{};
  const int rc = parse_pools(pools, 576 + 8, ks);
  if (rc != SMLA_OK) return rc;
  if (T > 0) {
    if (!pos || !cos_sin || !xo || !xo_scales) return fail(SMLA_EINVAL, "null pointer (pos, cos_sin, xo and xo_scales are required)");
    if (n_pos < 1) return fail(SMLA_EINVAL, "n_pos must be >= 1, got %d", n_pos);
    if (!aligned(pos, 4) || !aligned(cos_sin, 4) || !aligned(xo, 4) || !aligned(y_out, 16))
      return fail(SMLA_EINVAL, "pos, cos_sin and xo must be 4-byte aligned, y_out 16-byte aligned");
  }
  const V41Out v41{pos, cos_sin, n_pos, (uint8_t*)xo, (uint8_t*)xo_scales, y_out};
  return fwd_impl(q, q_stride_t, q_stride_h, ks, indptr, indices, nnz, T, H, sm_scale, has_invalid, sink,
                  nullptr, 0, 0, lse, workspace, workspace_bytes, stream, &v41);
}

int sparse_mla_mxfp8(const float* y, int64_t n, void* codes, void* scales, void* stream) {
  clear_err();
  if (n < 0 || n % 64 != 0) return fail(SMLA_EINVAL, "n must be a non-negative multiple of 64, got %lld", (long long)n);
  if (n == 0) return SMLA_OK;
  if (n / 512 + 1 > 0x7fffffff) return fail(SMLA_EINVAL, "n too large for one launch");
  if (!y || !codes || !scales) return fail(SMLA_EINVAL, "null pointer");
  if (!aligned(y, 4) || !aligned(codes, 8)) return fail(SMLA_EINVAL, "y must be 4-byte and codes 8-byte aligned");
  hipError_t e = smla::launch_mxfp8(y, n, (uint8_t*)codes, (uint8_t*)scales, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mxfp8 kernel launch");
  return SMLA_OK;
}

int sparse_mla_decode_rows(const void* kv, int64_t n_kv, const int32_t* rows, int64_t n,
                           float* out, void* stream) {
  clear_err();
  if (n < 0 || n_kv < 0) return fail(SMLA_EINVAL, "n and n_kv must be >= 0");
  if (n > 0x7fffffff) return fail(SMLA_EINVAL, "n too large for one launch");
  if (n == 0) return SMLA_OK;
  if (!kv || !rows || !out) return fail(SMLA_EINVAL, "null pointer");
  if (!aligned(kv, 16)) return fail(SMLA_EINVAL, "kv must be 16-byte aligned");
  hipError_t e = smla::launch_decode_rows((const uint8_t*)kv, n_kv, rows, n, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
  return SMLA_OK;
}

int sparse_mla_qk_probe(const void* q, const void* kv, int64_t n_kv, const int32_t* rows, int64_t n,
                        int32_t mode, float* scores, void* stream) {
  clear_err();
  if (n < 0 || n % 16 != 0) return fail(SMLA_EINVAL, "n must be a non-negative multiple of 16, got %lld", (long long)n);
  if (mode < 0 || mode > 3) return fail(SMLA_EINVAL, "mode must be 0, 1, 2 or 3, got %d", mode);
  if (n_kv < 1) return fail(SMLA_EINVAL, "n_kv must be >= 1");
  if (n / 16 > 0x7fffffff) return fail(SMLA_EINVAL, "n too large for one launch");
  if (n == 0) return SMLA_OK;
  if (!q || !kv || !rows || !scores) return fail(SMLA_EINVAL, "null pointer");
  if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(scores, 4)) return fail(SMLA_EINVAL, "q and kv must be 16-byte aligned");
  hipError_t e = smla::launch_qk_probe((const uint16_t*)q, (const uint8_t*)kv, n_kv, rows, n, mode, scores,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "qk probe kernel launch");
  return SMLA_OK;
}

int sparse_mla_cache_write(const void* latent, int64_t latent_stride,
                           const void* rope, int64_t rope_stride,
                           const int64_t* slots, int64_t n,
                           void* kv, int64_t n_kv, void* stream) {
  clear_err();
  if (n < 0 || n_kv < 0) return fail(SMLA_EINVAL, "n and n_kv must be >= 0");
  if (n_kv > INT64_MAX / smla::kRecordBytes) return fail(SMLA_EINVAL, "n_kv out of range: %lld", (long long)n_kv);
  if (n > (int64_t)0x7fffffff * 4) return fail(SMLA_EINVAL, "n too large for one launch");
  if (n == 0) return SMLA_OK;
  if (!latent || !rope || !slots || !kv) return fail(SMLA_EINVAL, "null pointer");
  if (!aligned(latent, 16) || !aligned(kv, 16) || !aligned(rope, 8) || !aligned(slots, 8))
    return fail(SMLA_EINVAL, "latent and kv must be 16-byte aligned, rope and slots 8-byte aligned");
  if (latent_stride < 512 || latent_stride % 8 != 0)
    return fail(SMLA_EINVAL, "latent_stride must be >= 512 and a multiple of 8 elements");
  if (rope_stride < 64 || rope_stride % 4 != 0)
    return fail(SMLA_EINVAL, "rope_stride must be >= 64 and a multiple of 4 elements");
  smla::CacheWriteParams p{(const uint16_t*)latent, latent_stride, (const uint16_t*)rope, rope_stride,
                           slots, n, (uint8_t*)kv, n_kv};
  hipError_t e = timed(3, [&](smla::Events ev) { return smla::launch_cache_write(p, ev, (hipStream_t)stream); });
  if (e != hipSuccess) return hip_fail(e, "cache writer launch");
  return SMLA_OK;
}

const char* sparse_mla_last_error(void) { return g_err; }

int sparse_mla_set_option(const char* name, int64_t value) {
  clear_err();
  if (!name) return fail(SMLA_EINVAL, "null option name");
  if (!strcmp(name, "plan")) {
    if (value < 0 || value > 2) return fail(SMLA_EINVAL, "plan must be 0, 1 or 2");
    g_plan_override.store(value, std::memory_order_relaxed);
    return SMLA_OK;
  }
  if (!strcmp(name, "persist")) {
    if (value < 0 || value > 1) return fail(SMLA_EINVAL, "persist must be 0 or 1");
    g_persist_override.store(value, std::memory_order_relaxed);
    return SMLA_OK;
  }
  if (!strcmp(name, "split")) {
    if (value < 0 || value > SMLA_MAX_SPLIT) return fail(SMLA_EINVAL, "split must be in [0, %d]", SMLA_MAX_SPLIT);
    g_split_override.store(value, std::memory_order_relaxed);
    return SMLA_OK;
  }
  return fail(SMLA_EINVAL, "unknown option '%s'", name);
}

int sparse_mla_profile_begin(int32_t max_calls) {
  clear_err();
  if (max_calls <= 0) return fail(SMLA_EINVAL, "max_calls must be > 0");
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (g_prof.active) return fail(SMLA_EINVAL, "profiling already active");
  const int pairs = SMLA_PROFILE_KINDS * max_calls;
  g_prof.ev.assign(2 * pairs, nullptr);
  g_prof.kind.assign(pairs, -1);
  for (auto& ev : g_prof.ev) {
    hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) {
      for (auto& x : g_prof.ev)
        if (x) (void)hipEventDestroy(x);
      g_prof.ev.clear();
      return hip_fail(e, "hipEventCreate");
    }
  }
  g_prof.cap = pairs;
  g_prof.used = 0;
  g_prof.active = true;
  return SMLA_OK;
}

int sparse_mla_profile_end(double* ms, int64_t* launches) {
  clear_err();
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.active) return fail(SMLA_EINVAL, "profiling not active");
  double acc[SMLA_PROFILE_KINDS] = {};
  int64_t cnt[SMLA_PROFILE_KINDS] = {};
  int rc = SMLA_OK;
  for (int i = 0; i < g_prof.used; ++i) {
    hipError_t e = hipEventSynchronize(g_prof.ev[2 * i + 1]);
    float t = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
    if (e != hipSuccess) {
      rc = hip_fail(e, "event timing");
      break;
    }
    const int k = g_prof.kind[i];
    acc[k] += t;
    cnt[k] += 1;
  }
  for (auto& x : g_prof.ev) (void)hipEventDestroy(x);
  g_prof.ev.clear();
  g_prof.kind.clear();
  g_prof.active = false;
  g_prof.cap = g_prof.used = 0;
  if (rc != SMLA_OK) return rc;
  for (int k = 0; k < SMLA_PROFILE_KINDS; ++k) {
    if (ms) ms[k] = acc[k];
    if (launches) launches[k] = cnt[k];
  }
  return SMLA_OK;
}

}  // extern "C"
