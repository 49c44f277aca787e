// Internal interface between the C ABI (smla_api.cpp) and the HIP kernels
// (smla_kernels.hip).  Not installed; the public ABI is include/smla.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

constexpr int kRecordBytes = 656;  // 512 e4m3 | 4 x f32 scale | 64 x bf16 rope
constexpr int kPlanBuckets = 256;   // longest-first counting-sort buckets (tiles, capped)

// Which index entries are keys.  Contiguous cache: entries >= 0.  Paged pools
// (K2-back page, key_rec): -1 is no key, an entry >= 0 a slot of pool 0 (the
// window pool), any other negative entry a slot of pool 1 (the compressed
// pool, slot = entry & 0x7fffffff); an entry of a pool that is absent is no key.
struct KeyMode {
  int32_t paged;
  int32_t present[2];
  __host__ __device__ bool valid(int32_t e) const {
    return paged ? (e != -1 && (e < 0 ? present[1] : present[0]) != 0) : e >= 0;
  }
};

struct PlanParams {
  const int32_t* indptr;
  const int32_t* indices;
  uint32_t idx_bytes;  // bytes of `indices` readable (bounded index reads)
  int32_t T;
  int32_t tile;        // tokens per tile
  int32_t has_invalid;
  KeyMode km;
  int32_t* row_tiles;  // [T] out: tiles of each row
  int32_t* order;      // [T] out: rows, longest first
  int32_t* desc;       // [T][4] out: slot r of the order as {row, slice start, length, tiles}
};

struct FwdParams {
  const uint16_t* q;   // bf16 bits
  int64_t q_st, q_sh;
  const uint8_t* kv;
  const uint8_t* zero; // a record of zeros on this device (masked positions read it)
  const int32_t* indptr;
  const int32_t* indices;
  uint32_t idx_bytes;
  int32_t T, H, S;     // rows, heads, chunks per row
  float c_log2;        // sm_scale * log2(e)
  uint16_t* out;       // bf16 bits
  int64_t o_st, o_sh;
  float* lse;          // nullable
  const int32_t* row_tiles;  // nullable: tiles from a scan of the slice (scan) or indptr
  int32_t scan;        // no plan and has_invalid: each block finds its row's last entry >= 0
  int32_t stride;      // > 0: no plan and every slice may start at row * stride (a guess the kernel checks)
  const int32_t* order;      // nullable: rows in their own order
  const int32_t* desc;       // with order: {row, slice start, length, tiles} of each rank (one load)
  uint16_t* part_o;    // f16 bits [T*S, H, 512] when S > 1 (dims permuted in 64-dim blocks: part_dim)
  float* part_lse;     // [T*S, H]  (log2 units) when S > 1
  KeyMode km;
  const uint8_t* pool[2];     // paged: page 0 of each pool
  int64_t pool_stride[2];     // paged: bytes from one page to the next
  int32_t pool_shift[2];      // paged: log2 of the records per page
  const float* sink;          // nullable: per-head sink logit [H] (natural log); unsplit rows only
  int32_t hg;                 // head groups per row (units per row = S * hg)
  int32_t persist;            // > 0: blocks of a persistent grid (a multiple of 8, one per CU), for
                              // kernels that run several units per block; 0: one unit per block
};

struct CombineParams {
  int32_t T, H, S;
  const float* sink;     // nullable: per-head sink logit [H] (natural log)
  const int32_t* order;  // nullable: rows in their own order
  const uint16_t* part_o;  // f16 bits
  const float* part_lse;
  uint16_t* out;
  int64_t o_st, o_sh;
  float* lse;
};

// The V4.1 record's combine and output epilogue (smla_v41.hip).
struct Combine41Params {
  int32_t T, H, S;
  const float* sink;       // nullable: per-head sink logit [H] (natural log)
  const int32_t* order;    // nullable: rank -> row
  const uint16_t* part_o;  // f16 bits [T*S, H, 512] (every row has partials)
  const float* part_lse;   // [T*S, H] log2 units
  const int32_t* pos;      // [T] position of each row (clamped to [0, n_pos))
  const float* cos_sin;    // [n_pos, 64]: 32 cos, then 32 sin
  int32_t n_pos;
  uint8_t* xo;             // [T, H, 512] E4M3 codes
  uint8_t* xos;            // [T, H, 16] E8M0 bytes, one per 32 dims
  float* lse;              // nullable: [T, H] natural log, sink included
  float* y_out;            // nullable: [T, H, 512] the values quantised (checking)
};

struct CacheWriteParams {
  const uint16_t* latent;  // bf16 bits [n, 512], row stride latent_st elements
  int64_t latent_st;
  const uint16_t* rope;    // bf16 bits [n, 64], row stride rope_st elements
  int64_t rope_st;
  const int64_t* slots;    // [n]: record index of token i; < 0 or >= n_kv: not written
  int64_t n;
  uint8_t* kv;             // [n_kv, 656]
  int64_t n_kv;
};

// Head tiling: tiles of 16 heads.  Tokens per tile: 128 for the H <= 16
// kernel, 64 for the 17..32-head kernel, 32 for the kernel above 32 heads.
inline int head_tiles(int H) { return (H + 15) / 16; }
inline int tile_tokens(int H) { return head_tiles(H) == 1 ? 128 : head_tiles(H) == 2 ? 64 : 32; }
// Head groups of a row: the wide-head kernel takes at most 64 heads per unit.
inline int head_groups(int H) { return (H + 63) / 64; }

// Optional timing events: `start` is attached to the first kernel dispatch of
// a launch and `stop` to the last (hipExtLaunchKernel); null = untimed.
struct Events {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// The has_invalid scan (row_tiles) when p.has_invalid; the longest-first sort
// (order, and row_tiles from indptr when there was no scan) when `sort`.
hipError_t launch_plan(const PlanParams& p, bool sort, Events ev, hipStream_t s);
hipError_t launch_fwd(const FwdParams& p, Events ev, hipStream_t s);
// The wide-head forward: 17 <= H <= 32 (smla_wide.hip), above 32 heads the
// kernel of smla_wide64.hip (launch_fwd_wide64).
hipError_t launch_fwd_wide(const FwdParams& p, Events ev, hipStream_t s);
hipError_t launch_fwd_wide64(const FwdParams& p, Events ev, hipStream_t s);
// Device address of the library's zero record on the current device.
hipError_t zero_record_address(const uint8_t** out);
hipError_t launch_combine(const CombineParams& p, Events ev, hipStream_t s);
hipError_t launch_cache_write(const CacheWriteParams& p, Events ev, hipStream_t s);
// V4.1 records (H <= 16): forward partials, then the combine + epilogue.
hipError_t launch_fwd41(const FwdParams& p, Events ev, hipStream_t s);
hipError_t launch_combine41(const Combine41Params& p, Events ev, hipStream_t s);
// Test hook: MXFP8 of n f32 values (n a multiple of 64).
hipError_t launch_mxfp8(const float* y, int64_t n, uint8_t* codes, uint8_t* scales, hipStream_t s);
// Device address of the static scratch of sparse_mla_fwd_noalloc on device
// dev (looked up once per device with that device current; smla_noalloc.hip).
hipError_t noalloc_scratch(int dev, void** out);
// Test hook (smla_qk_probe.hip): QK scores of n tokens (n a multiple of 16)
// against 16 heads, by the forward's bf16 path (mode 0) or the scaled fp8
// MFMA with the q hi/lo split (mode 1; mode 2: hi only).
hipError_t launch_qk_probe(const uint16_t* q, const uint8_t* kv, int64_t n_kv, const int32_t* rows, int64_t n,
                           int mode, float* scores, hipStream_t s);
hipError_t launch_decode_rows(const uint8_t* kv, int64_t n_kv, const int32_t* rows, int64_t n,
                              float* out, hipStream_t s);

// Blocks a launch of T rows x `per_row` blocks uses with the XCD-aware mapping.
inline int64_t xcd_grid(int32_t T, int32_t per_row) { return 8LL * ((T + 7) / 8) * per_row; }
// Blocks of the split forward's unit mapping (fwd_unit, smla_device.h).
inline int64_t fwd_grid(int32_t T, int32_t S, bool ranged) {
  if (ranged && (S == 2 || S == 4 || S == 8)) {
    const int G = 8 / S;
    return 8LL * ((T + G - 1) / G);
  }
  if (ranged && (S == 16 || S == 32)) return (int64_t)T * S;
  return xcd_grid(T, S);
}

}  // namespace smla
