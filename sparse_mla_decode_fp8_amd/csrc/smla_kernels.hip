// HIP kernels for sparse MLA forward over fp8_ds_mla records, CDNA4 (gfx950).
//
// Method (vLLM API page "vllm.models.kimi_k3.amd.ops.flydsl_sparse_mla_gfx950",
// module docstring): each query row attends to the KV records of its CSR slice;
// K is the decoded 576-value record, V its 512 latent values; the softmax is
// online over tiles of the slice, with P = exp2(x - m + 8) so that P <= 2^8 and
// P times a V scale <= 2^7 still fits f16.  The split of long rows into chunks
// merged by their (max, sum) follows the K2-back page
// ("vllm.models.deepseek_v41.amd.mono.attention.back", module docstring and
// stage_combine).
//
// Design for MI355X (this file: plan, the H <= 16 forward, combine, record
// writer and decode hook; the wide-head forward is smla_wide.hip):
//  * plan kernels: per-row tile counts (a bounded scan for the last valid
//    entry when has_invalid) and a longest-first row order (counting sort),
//    launched only when there are more units than compute units.
//  * forward kernel: a workgroup owns one (row, chunk) unit.  Records arrive
//    by LDS DMA (global_load_lds_dwordx4 from 64-bit per-lane record
//    addresses) two tiles deep; masked positions read a zero record.
//  * QK: K dequantised exactly to bf16 by v_cvt_scalef32_pk_bf16_fp8 with the
//    record's pow2 scale (the conversion applies the scale's exponent only),
//    bf16 MFMA 16x16x32 against bf16 q held in registers (rope the same).
//  * PV: V read transposed from LDS (ds_read_b64_tr_b8), converted exactly
//    e4m3 -> f16, f16 MFMA 16x16x32; the per-token V scale is folded into P,
//    which passes between waves through LDS.
//  * combine kernel: LSE merge of the chunks of split rows (with the sink).
//  * workgroup -> unit mapping is XCD-aware (dispatch is round-robin over the
//    8 XCDs): chunk c of every split row runs on the same XCDs, so rows whose
//    sorted slices share records share them through that XCD's L2 (fwd_unit).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "smla_device.h"

namespace smla {

// A record of zeros: masked positions gather it, so they read finite data
// (V = 0, scale = 0) wherever the cache is, and never address row 0.
__device__ __attribute__((aligned(256))) uint8_t g_zero_record[kRecordBytes];

// ---------------------------------------------------------------- plan

// has_invalid only: one 256-thread block per row finds 1 + the last slice
// position whose entry is a key (bounded index reads, 2048 entries a round
// with every load issued before any is used) and stores the row's tile count.
// (indptr, indices and their size are preloaded leading arguments)
__global__ __launch_bounds__(256) void smla_plan_scan_kernel(
    const int32_t* __restrict__ indptr, const int32_t* __restrict__ indices, uint32_t idx_bytes, PlanParams p) {
  __shared__ int s_red[4];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int beg = indptr[row];
  const int len = max(indptr[row + 1] - beg, 0);
  const __amdgpu_buffer_rsrc_t r = idx_rsrc(indices, idx_bytes);
  int lastp = 0;
  for (int base = 0; base < len; base += 8 * 256) {
    int v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = load_idx(r, (uint32_t)(beg + base + 256 * j + tid) * 4u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int pos = base + 256 * j + tid;
      if (pos < len && p.km.valid(v[j])) lastp = max(lastp, pos + 1);
    }
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) lastp = max(lastp, __shfl_xor(lastp, sh));
  if ((tid & 63) == 0) s_red[tid >> 6] = lastp;
  __syncthreads();
  if (tid == 0) p.row_tiles[row] = tiles_of(max(max(s_red[0], s_red[1]), max(s_red[2], s_red[3])), p.tile);
}

// Adds one per active lane to cnt[b] and returns each active lane's slot (the
// old count plus its rank among the wave's lanes with the same b).  When every
// active lane of the wave has the same b (equal-length rows) that is one LDS
// atomic for the wave instead of one per lane on a single address; otherwise
// one atomic per lane.  Wave-uniform control flow.
__device__ __forceinline__ int wave_bucket_add(int* cnt, int b, bool active) {
  const int lane = threadIdx.x & 63;
  const uint64_t act = __ballot(active);
  if (!act) return 0;
  const int leader = __builtin_ctzll(act);
  const int lb = __shfl(b, leader);
  if (__ballot(active && b == lb) == act) {
    int base = 0;
    if (lane == leader) base = atomicAdd(&cnt[lb], (int)__popcll(act));
    base = __shfl(base, leader);
    return base + (int)__popcll(act & ((1ull << lane) - 1));
  }
  return active ? atomicAdd(&cnt[b], 1) : 0;
}

// One block: tile counts of every row (from the scan, or from indptr) and a
// counting sort of the rows by tile count, longest first (the FlyDSL page
// issues long rows first so the long tail starts early).  Each slot of the
// order also gets its row's {row, slice start, length, tiles}, so that a
// forward block finds its unit with one load instead of two in a row.
// (the row tiles, indptr, T and has_invalid are preloaded leading arguments)
__global__ __launch_bounds__(1024) void smla_plan_sort_kernel(
    int32_t* __restrict__ row_tiles, const int32_t* __restrict__ indptr, int32_t T, int32_t has_invalid,
    PlanParams p) {
  __shared__ int s_cnt[kPlanBuckets];
  __shared__ int s_wsum[kPlanBuckets / 64];
  const int tid = threadIdx.x;
  for (int i = tid; i < kPlanBuckets; i += blockDim.x) s_cnt[i] = 0;
  __syncthreads();
  // (every thread runs the same number of rounds: the wave-wide steps need
  // whole waves)
  for (int r0 = 0; r0 < T; r0 += blockDim.x) {
    const int r = r0 + tid;
    int t = 0;
    if (r < T) {
      if (has_invalid) {
        t = row_tiles[r];
      } else {
        t = tiles_of(max(indptr[r + 1] - indptr[r], 0), p.tile);
        row_tiles[r] = t;
      }
    }
    wave_bucket_add(s_cnt, min(t, kPlanBuckets - 1), r < T);
  }
  __syncthreads();
  // exclusive prefix over buckets in descending order: start[b] = sum_{b' > b} cnt[b'].
  // Threads < kPlanBuckets (whole waves) scan; every thread meets every barrier.
  const bool scanner = tid < kPlanBuckets;
  const int b = kPlanBuckets - 1 - (scanner ? tid : 0);  // position tid in descending order
  const int c = scanner ? s_cnt[b] : 0;
  int incl = c;
  if (scanner) {
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      const int o = __shfl_up(incl, sh);
      if ((tid & 63) >= sh) incl += o;
    }
    if ((tid & 63) == 63) s_wsum[tid >> 6] = incl;
  }
  __syncthreads();
  if (scanner) {
    int off = 0;
    for (int w = 0; w < (tid >> 6); ++w) off += s_wsum[w];
    s_cnt[b] = off + incl - c;
  }
  __syncthreads();
  for (int r0 = 0; r0 < T; r0 += blockDim.x) {
    const int r = r0 + tid;
    const int t = r < T ? row_tiles[r] : 0;
    const int beg = r < T ? indptr[r] : 0;
    const int end = r < T ? indptr[r + 1] : 0;
    const int slot = wave_bucket_add(s_cnt, min(t, kPlanBuckets - 1), r < T);
    if (r < T) {
      p.order[slot] = r;
      // the forward blocks take their unit in one load
      *(v4i*)(p.desc + 4 * slot) = v4i{r, beg, max(end - beg, 0), t};
    }
  }
}

// ---------------------------------------------------------------- forward, H <= 16

// One block of 8 waves (two per SIMD) per unit; tiles of 128 tokens.
//   QK: wave w scores tokens 16w .. 16w+15 of the tile for all 16 heads.
//   PV: wave w accumulates output dims 64w .. 64w+63 (half a scale block, so
//       the V scale folds into P) over all 128 tokens, and the softmax sum of
//       every head from the same f16 P it multiplies.
// P, the per-token V scales and the per-wave tile maxima go through LDS, with
// two barriers per tile; no merge is needed at the end.
//
// Pipeline: two latent stages.  Tile n+2 is queued into tile n's stage as soon
// as every wave has finished tile n, so while a wave waits for tile n+1 both
// n+1 and n+2 are in flight.  Each wave's QK reads only the records its own
// DMA brought in, so a wave starts tile n after its own wait; the barrier
// after the scores publishes every wave's records for the P.V stage.  The
// scales and rope a lane needs for QK travel with the records into one of two
// register sets (tiles alternate between them, so the loop is unrolled by
// two).
namespace n16 {
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 128;
constexpr int kPair = 2 * kLat + 16;             // two latent rows + 16-B pad
constexpr int kLatStage = (kTile / 2) * kPair;   // 66560 B
constexpr int kIdxRing = 4;                      // index ring slots (tiles)
constexpr int kLatOff = 0;
// Rows of q, P and the V scales are padded by 16 bytes so that the rows of
// different heads (blocks) start on different LDS banks: the reads of one
// instruction then spread over all banks instead of piling onto the same few.
constexpr int kQRow = 2 * 576 + 16;               // 1168 B
constexpr int kPRow = 2 * kTile + 16;             // 272 B
constexpr int kQOff = kLatOff + 2 * kLatStage;    // q of the row, bf16 [head 16][576 (+pad)]
constexpr int kPxOff = kQOff + 16 * kQRow;        // P, f16 [head 16][token 128 (+pad)]
constexpr int kSxOff = kPxOff + 16 * kPRow;       // V scales, f16 [block 4][token 128 (+pad)]
constexpr int kMxOff = kSxOff + 4 * kPRow;        // tile maxima, f32 [head 16][wave 8]
constexpr int kIdxRingOff = kMxOff + 16 * kWaves * 4;
constexpr int kTabOff = kIdxRingOff + kIdxRing * kTile * 4;  // record addresses [2][token 128]
constexpr int kBytes = kTabOff + 2 * kTile * 8;
static_assert(kBytes <= 160 * 1024, "LDS budget");
constexpr int kOutPitch = 2 * 64 + 16;            // epilogue staging row: 64 bf16 dims + pad
static_assert(kWaves * 16 * kOutPitch <= 16 * kQRow, "epilogue staging fits the q area");
// Vector-memory instructions one wave issues per tile: 8 latent DMAs (token
// pairs) and 3 side loads; one index DMA per tile besides.
constexpr int kTileVm = 8 + 3;

// Byte offset of token tau's latent row inside a stage.  Rows come in pairs
// (2 x 512 B, then a 16-B pad); the odd row of a pair stores chunk c (16 B)
// at position c ^ 8.  With the 1040-B pair stride both the QK reads (16
// tokens, one chunk column) and the transposed PV reads spread over all banks.
__device__ __forceinline__ uint32_t row_off(int tau) { return (tau >> 1) * kPair + (tau & 1) * kLat; }

// Scales and rope of the token a lane scores (token 16w + t): the 4 block
// scales, rope dims 8g .. 8g+7 and 32 + 8g .. 32 + 8g + 7; and the wave's
// valid-token mask of that tile (bit j: token 16w + j is a key).
struct Side {
  v4f ksc;
  v4i rp0, rp1;
  uint32_t vmask;
};

// After the wait that covers a side load: later reads of the registers may
// not move above this point.
__device__ __forceinline__ void pin(Side& s) { asm volatile("" : "+v"(s.ksc), "+v"(s.rp0), "+v"(s.rp1)); }

}  // namespace n16

// The fields the prologue needs first come as separate scalar arguments ahead
// of the parameter block, so that they are preloaded into SGPRs at wave
// launch instead of waiting for a load of the kernel arguments.  `stride`
// (> 0) is the slice stride nnz / T when there is no plan and nnz divides
// evenly: each block then guesses its slice start (rank * stride) and queues
// its first index tiles before indptr arrives, and queues them again from the
// real start if the guess was wrong.
// MULTI (with the plan only): a persistent grid of a multiple of 8 blocks, at
// most one per CU.  In round k block b runs the unit of virtual block
// k * grid + b of the one-unit-per-block grid, or in odd rounds that of b
// mirrored among its XCD's blocks, so that in the longest-first order a
// block's units pair long with short, each on the XCD the plain grid would
// use.  A unit loads the next one's descriptor after its own first loads and
// queues the next one's first index tiles after its last tile, so the next
// unit starts with both at hand.
template <bool MULTI>
__global__ __launch_bounds__(n16::kThreads, 1) void smla_fwd16_kernel(
    const int32_t* __restrict__ indptr, const int32_t* __restrict__ indices, const uint16_t* __restrict__ qbase,
    const int32_t* __restrict__ desc, int32_t T, int32_t S, uint32_t idx_bytes, int32_t stride, FwdParams p) {
  using namespace n16;
  __shared__ __attribute__((aligned(1024))) uint8_t s_lds[kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 15;
  const int g = lane >> 4;

  // (persistent) the parameter block read at a unit's start and end comes
  // through a pointer the compiler cannot see through (the kernel arguments in
  // their segment: the leading scalars, then the block at its natural
  // alignment), so its fields are loaded where they are used instead of being
  // held in registers through every unit's tiles
  struct KArgs {
    const int32_t* indptr;
    const int32_t* indices;
    const uint16_t* qbase;
    const int32_t* desc;
    int32_t T, S;
    uint32_t idx_bytes;
    int32_t stride;
    FwdParams p;
  };
  static_assert(offsetof(KArgs, p) == 48, "the parameter block follows the 48 bytes of leading arguments");
  typedef const __attribute__((address_space(4))) KArgs* KArgsP;
  auto pa = [&]() -> const __attribute__((address_space(4))) FwdParams* {
    KArgsP a = (KArgsP)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(a));
    return &a->p;
  };
#define SMLA_P(f) (MULTI ? pa()->f : p.f)

  int rank, chunk;
  fwd_unit(S, desc == nullptr, rank, chunk);
  // (persistent) the block's first unit after round kr that holds a row
  int kr = 0;
  auto next_rank = [&](int& r, int& c) -> bool {
    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    const int mirror = (b & 7) + 8 * (G / 8 - 1 - (b >> 3));
    const int nvb = 8 * ((T + 7) / 8) * S;
    for (++kr; kr * G < nvb; ++kr) {
      const int v = kr * G + ((kr & 1) ? mirror : b);
      if (v >= nvb) continue;
      xcd_unit_at(v, S, r, c);
      if (r < T) return true;
    }
    return false;
  };
  if (rank >= T && !(MULTI && next_rank(rank, chunk))) return;

  const uint32_t base = lds_addr(s_lds);
  const __amdgpu_buffer_rsrc_t irs = idx_rsrc(indices, idx_bytes);
  auto ring_at = [&](int n) -> uint32_t { return base + kIdxRingOff + (n & (kIdxRing - 1)) * kTile * 4; };
  // index DMA of tile n of the slice starting at b: this wave's 16 entries
  // (lanes 0..15).  Positions past nnz read 0 (bounded reads); positions past
  // the row are masked in fill_table.
  auto issue_idx_at = [&](int b, int n) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(ring_at(n) + 64 * w);
    if (lane < 16) buf_dma4(irs, (uint32_t)(b + n * kTile + 16 * w + lane) * 4u, dst);
  };
  // speculative start (no plan: row = rank)
  const int beg_g = rank * stride;
  const int tiles_g = (stride + kTile - 1) / kTile;
  const int t0_g = min(chunk * ((tiles_g + S - 1) / S), tiles_g);
  if (stride > 0) {
    issue_idx_at(beg_g, t0_g);
    issue_idx_at(beg_g, t0_g + 1);
    issue_idx_at(beg_g, t0_g + 2);
  }

  // (persistent) the next unit, and its descriptor (lane i holds field i & 3;
  // an ordinary load, whose wait the compiler places); have_ud: this unit's
  // descriptor came from the unit before; pref: so did its first index tiles
  int rank_n = 0, chunk_n = 0;
  bool have_ud = false, pref = false;
  int ud_n = 0;
  for (;;) {
    // (persistent) lane-derived values are formed anew in each unit, from an
    // opaque copy of the lane index, instead of being held across units
    int lane_u = lane;
    if (MULTI) asm volatile("" : "+v"(lane_u));
    const int lane = lane_u, t = lane & 15, g = lane >> 4;
    int row, beg, len, tiles;
    if (MULTI && have_ud) {
      row = __builtin_amdgcn_readlane(ud_n, 0);
      beg = __builtin_amdgcn_readlane(ud_n, 1);
      len = __builtin_amdgcn_readlane(ud_n, 2);
      tiles = __builtin_amdgcn_readlane(ud_n, 3);
    } else if (desc) {  // with the plan, the unit of rank `rank` in one load
      const v4i ud = *(const v4i*)(desc + 4 * rank);
      row = ud.x;
      beg = ud.y;
      len = ud.z;
      tiles = ud.w;
    } else {
      row = rank;
      beg = indptr[row];
      len = max(indptr[row + 1] - beg, 0);
      tiles = unit_tiles<kThreads>(p, row, beg, len, kTile, (int*)(s_lds + kMxOff));
    }
    const int ct = (tiles + S - 1) / S;
    const int t0 = min(chunk * ct, tiles);
    const int t1 = min(t0 + ct, tiles);
    const int unit = row * S + chunk;
    const bool split = S > 1;
    const int H = SMLA_P(H);
    const int h = t;  // head of this lane in QK (C column) and PV (B column)
    const bool h_ok = h < H;
    const bool has_n = MULTI && next_rank(rank_n, chunk_n);

    if (t0 >= t1) {  // nothing to attend: zero output and the sink's lse, or an empty partial
      if (stride > 0 || pref) wait_vm_all();  // the speculative or queued index DMAs land before the block ends
      if (split) {
        for (int hh = tid; hh < H; hh += kThreads) SMLA_P(part_lse)[(int64_t)unit * H + hh] = -INFINITY;
      } else {
        for (int e = tid; e < H * (kLat / 8); e += kThreads) {
          const int hh = e / (kLat / 8), d = (e % (kLat / 8)) * 8;
          *(v4i*)(SMLA_P(out) + row * SMLA_P(o_st) + hh * SMLA_P(o_sh) + d) = v4i{0, 0, 0, 0};
        }
        float* const lse_o = SMLA_P(lse);
        const float* const sink_o = SMLA_P(sink);
        if (lse_o)  // a row with no key: lse is the sink (-inf without one)
          for (int hh = tid; hh < H; hh += kThreads)
            lse_o[(int64_t)row * H + hh] = sink_o ? sink_o[hh] : -INFINITY;
      }
      if (!has_n) return;
      ud_n = desc[4 * rank_n + (lane & 3)];
      rank = rank_n;
      chunk = chunk_n;
      have_ud = true;
      pref = false;
      continue;
    }

    const uint8_t* const kv = p.kv;
    const uint8_t* const zero = p.zero;
    auto lat_at = [&](int st) -> uint32_t { return base + kLatOff + st * kLatStage; };
    auto tab_at = [&](int n) -> uint32_t { return base + kTabOff + (n & 1) * kTile * 8; };
    // Every wave touches only its own 16 entries of the index ring and the
    // address table, so those need no barrier.
    auto issue_idx = [&](int n) { issue_idx_at(beg, n); };
    // record addresses of this wave's tokens of tile n (masked ones: the zero
    // record); returns the wave's valid-token mask
    auto fill_table = [&](int n) -> uint32_t {
      int ix = -1;
      if (lane < 16) {
        const int raw = *LDSP(int, ring_at(n) + 4 * (16 * w + lane));
        ix = (n * kTile + 16 * w + lane < len) ? raw : -1;
        *LDSP(uint64_t, tab_at(n) + 8 * (16 * w + lane)) =
            (uint64_t)(uintptr_t)(p.km.valid(ix) ? key_addr(p, ix) : zero);
      }
      return (uint32_t)__ballot(lane < 16 && p.km.valid(ix)) & 0xFFFFu;
    };
    // latent DMA of this wave's 16 tokens of tile n into stage st: one
    // instruction per token pair, lanes 0..31 the even token, 32..63 the odd one
    // (lane position p of the odd row loads chunk p ^ 8).
    const uint32_t src_chunk = 16u * (uint32_t)((lane & 31) ^ ((lane >> 5) << 3));
    auto issue_latent = [&](int n, int st) {
      const uint32_t tab = tab_at(n) + 8 * (16 * w + (lane >> 5));
      uint64_t a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = *LDSP(uint64_t, tab + 16 * i);
      const uint32_t dst = lat_at(st) + 8 * w * kPair;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dma16((const uint8_t*)(uintptr_t)(a[i] + src_chunk), __builtin_amdgcn_readfirstlane(dst + i * kPair));
    };
    auto load_side = [&](int n, Side& s) {
      const uint64_t rec = *LDSP(uint64_t, tab_at(n) + 8 * (16 * w + t));
      gload16(s.ksc, rec + kScaleOff);
      gload16(s.rp0, rec + kRopeOff + 16 * g);
      gload16(s.rp1, rec + kRopeOff + 64 + 16 * g);
    };
    // Tile n's loads with every address already in registers: fill_table(n)
    // and the table reads run while an earlier tile is processed, so that the
    // refill after a tile only issues loads.
    struct Next {
      uint64_t lat[8];  // latent DMA source rows (issue_latent's a[])
      uint64_t rec;     // the side loads' record (load_side's rec)
      uint32_t vmask;
    };
    auto prep = [&](int n, Next& nx) {
      nx.vmask = fill_table(n);
      const uint32_t tab = tab_at(n) + 8 * (16 * w + (lane >> 5));
#pragma unroll
      for (int i = 0; i < 8; ++i) nx.lat[i] = *LDSP(uint64_t, tab + 16 * i);
      nx.rec = *LDSP(uint64_t, tab_at(n) + 8 * (16 * w + t));
    };
    auto issue_next = [&](const Next& nx, int st, Side& s) {
      const uint32_t dst = lat_at(st) + 8 * w * kPair;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dma16((const uint8_t*)(uintptr_t)(nx.lat[i] + src_chunk), __builtin_amdgcn_readfirstlane(dst + i * kPair));
      gload16(s.ksc, nx.rec + kScaleOff);
      gload16(s.rp0, nx.rec + kRopeOff + 16 * g);
      gload16(s.rp1, nx.rec + kRopeOff + 64 + 16 * g);
      s.vmask = nx.vmask;
    };

    // ---- prologue.  q of the row into LDS (each wave an eighth, once per
    // block) alongside the first three index tiles; then the first two tiles'
    // records, with index tiles t0+3 and t0+4 queued as if by iterations
    // t0-2 and t0-1, so every iteration sees the same order of loads:
    //   ... S(n) | I(n+3) | L(n+1) S(n+1) | I(n+4) ...
    // (L latent DMA, S side loads, I index DMA of a tile).
    // index tiles t0 .. t0+2, unless the speculative ones are those
    if (!pref && !(stride > 0 && beg == beg_g && t0 == t0_g)) {
      if (stride > 0) wait_vm_all();  // the guessed tiles land before the ring is refilled
      issue_idx(t0);
      issue_idx(t0 + 1);
      issue_idx(t0 + 2);
    }
    // wave w loads q heads 2w and 2w+1: chunk c (16 B, 72 per head) of head hh
    // lands at q_lds + kQRow hh + 16 c; heads >= H are not loaded (their lanes
    // use zeros).  nq: q DMA instructions this wave issues.
    const int nq = 2 * ((2 * w < H) + (2 * w + 1 < H));
    {
      const uint16_t* qrow = qbase + row * SMLA_P(q_st);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int hh = 2 * w + j;
        if (hh < H) {
          const uint16_t* qh = qrow + (int64_t)hh * SMLA_P(q_sh);
          const uint32_t dst = base + kQOff + kQRow * hh;
          dma16((const uint8_t*)(qh + 8 * lane), __builtin_amdgcn_readfirstlane(dst));
          if (lane < 8) dma16((const uint8_t*)(qh + 8 * (64 + lane)), __builtin_amdgcn_readfirstlane(dst + 1024));
        }
      }
    }
    // this wave's index tiles have landed (its q chunks may still be in flight)
    if (nq == 4) wait_vm<4>();
    else if (nq == 2) wait_vm<2>();
    else wait_vm<0>();
    Side sA, sB;    // tiles t0, t0+2, ... use sA; t0+1, t0+3, ... sB
    sA.vmask = fill_table(t0);
    sB.vmask = (t0 + 1 < t1) ? fill_table(t0 + 1) : 0u;
    issue_latent(t0, 0);
    load_side(t0, sA);
    // Index tiles past the unit's end are never queued (from here on), so
    // none is left in flight when the block ends.
    if (t0 + 3 < t1) {
      issue_idx(t0 + 3);
      wait_vm<kTileVm + 1>();  // this wave's q chunks have landed (tile t0 and I(t0+3) may not)
    } else {
      wait_vm<kTileVm>();
    }
    __syncthreads();  // every wave's q chunks have landed
    // (persistent) the next unit's descriptor, behind this unit's first loads
    if (MULTI && has_n) ud_n = desc[4 * rank_n + (lane & 3)];
    // q as bf16 B operands (head = lane column t).  Latent K-step 2m / 2m+1: dims
    // 64m + 16g + [0..7] / [8..15]; rope K-step i: dims 512 + 32i + 8g + [0..7].
    v8bf qlat[16];
    v8bf qrope[2];
    {
      const uint32_t qr = base + kQOff + kQRow * t;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        v4i a = *LDSP(v4i, qr + 2 * (64 * m + 16 * g));
        v4i b = *LDSP(v4i, qr + 2 * (64 * m + 16 * g + 8));
        if (!h_ok) a = b = v4i{0, 0, 0, 0};
        qlat[2 * m] = __builtin_bit_cast(v8bf, a);
        qlat[2 * m + 1] = __builtin_bit_cast(v8bf, b);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        v4i a = *LDSP(v4i, qr + 2 * (kLat + 32 * i + 8 * g));
        if (!h_ok) a = v4i{0, 0, 0, 0};
        qrope[i] = __builtin_bit_cast(v8bf, a);
      }
    }

    float m_ref = -INFINITY;  // reference max (log2 units), the same in every wave
    float l_run = 0.0f;       // head t's sum of P over this lane's tokens (PV side)
    v4f O[4];                 // O^T slices: dims 64w + 16 dt + 4g + [0..3], head t
#pragma unroll
    for (int i = 0; i < 4; ++i) O[i] = v4f{0, 0, 0, 0};

    // QK read addresses: token 16w + t, chunk 4m + g (stored at (4m + g) ^ 8 in odd rows,
    // i.e. K-step m ^ 2): slices with m & 2 == 0 use qk_a, the others qk_b, + 64 m.
    const uint32_t qk_row = row_off(16 * w + t) + 16 * g;
    const uint32_t qk_a = qk_row + ((t & 1) ? 128u : 0u);
    const uint32_t qk_b = qk_row - ((t & 1) ? 128u : 0u);
    // PV transposed reads: lane (t, g) loads token 32 k + 8 g + t/2, bytes
    // 8(t&1) .. +7 of chunk 4w + dt (stored at (4w + dt) ^ 8 in odd rows), so
    // lane (i, g) receives dim i of tokens 8g .. 8g+7 of K-step k; dt and k are
    // immediate offsets.
    const int tv = 8 * g + (t >> 1);
    const uint32_t pv_off = row_off(tv) + 64 * (w ^ (2 * (tv & 1))) + 8 * (t & 1);
    const v2h ones = v2h{(_Float16)1.0f, (_Float16)1.0f};

    const uint32_t mx = base + kMxOff;
    const uint32_t px = base + kPxOff;
    const uint32_t sx = base + kSxOff;
    Next nx;

    // One tile: n, its stage st (= (n - t0) & 1) and its side registers.
    auto tile = [&](int n, int st, Side& sd) __attribute__((always_inline)) {
      // this wave's records, scales and rope of tile n have landed; the loads
      // queued after them (I(n+3), tile n+1's, I(n+4), each only if that tile
      // exists) may still be in flight.  Tile t0 alone is queued by itself
      // (followed by I(t0+3) only), so that the first records of every block
      // arrive as early as they can; tile t0+1 follows as soon as they have.
      const int left = t1 - n;  // tiles left, this one included
      if (n == t0) {
        // (after I(t0+3) if queued, and the next unit's descriptor if loaded)
        if (MULTI && has_n) {
          if (left >= 4) wait_vm<2>();
          else wait_vm<1>();
        } else {
          if (left >= 4) wait_vm<1>();
          else wait_vm<0>();
        }
        if (left >= 2) {
          issue_latent(n + 1, st ^ 1);
          load_side(n + 1, sB);
        }
        if (left >= 5) {
          __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // ring slot t0 was read before I(t0+4) lands in it
          issue_idx(n + 4);
        }
      } else if (left >= 5) {
        wait_vm<2 + kTileVm>();
      } else if (left == 4) {
        wait_vm<1 + kTileVm>();
      } else if (left >= 2) {
        wait_vm<kTileVm>();
      } else {
        wait_vm<0>();
      }
      pin(sd);

      // ---- QK: lane (t, g) gets head t, tokens 16w + 4g + r (own records only)
      const uint32_t lat = lat_at(st);
      v4f S;
      {
        v4i kr[8];
#pragma unroll
        for (int m = 0; m < 8; ++m) kr[m] = *LDSP(v4i, lat + ((m & 2) ? qk_b : qk_a) + 64 * m);
        // all eight reads are issued before the first conversion waits for one
        // (left to itself the scheduler issues them in pairs, each pair waited for)
        __builtin_amdgcn_sched_barrier(0);
        // two independent accumulation chains (K-steps 2m and 2m+1), summed at the end
        v4f acc0 = v4f{0, 0, 0, 0}, acc1 = v4f{0, 0, 0, 0};
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, sd.rp0), qrope[0], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, sd.rp1), qrope[1], acc1, 0, 0, 0);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float sc = sd.ksc[m >> 1];
          v2bf a0, a1, a2, a3, b0, b1, b2, b3;
          cvt4_bf16(kr[m].x, sc, a0, a1);
          cvt4_bf16(kr[m].y, sc, a2, a3);
          cvt4_bf16(kr[m].z, sc, b0, b1);
          cvt4_bf16(kr[m].w, sc, b2, b3);
          const v8bf ka = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
          const v8bf kb = {b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qlat[2 * m], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qlat[2 * m + 1], acc1, 0, 0, 0);
        }
        S = acc0 + acc1;
      }

      // ---- softmax (log2 domain) of this wave's 16 tokens
      float x[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = ((sd.vmask >> (4 * g + r)) & 1u) ? S[r] * p.c_log2 : -INFINITY;
        tmax = fmax_(tmax, x[r]);
      }
      tmax = xor_max(tmax);
      if (g == 0) *LDSP(float, mx + 4 * (8 * t + w)) = tmax;
      // P with the current reference (valid unless some head's max moves it)
      auto write_p = [&](float m_use) {
        _Float16 ph[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ph[r] = (_Float16)__builtin_amdgcn_exp2f(x[r] - m_use + kShift);
        *LDSP(v2i, px + kPRow * t + 2 * (16 * w + 4 * g)) =
            __builtin_bit_cast(v2i, (v4h{ph[0], ph[1], ph[2], ph[3]}));
      };
      write_p(m_ref == -INFINITY ? 0.0f : m_ref);
      // V scale of block g for token 16w + t, clamped to 2^7, as f16
      *LDSP(_Float16, sx + kPRow * g + 2 * (16 * w + t)) = (_Float16)__builtin_fminf(sd.ksc[g], kScaleCap);
      // tile n+2's addresses, while the other waves' records may still be
      // landing: its index tile was queued before tile n's records (which have
      // landed), table slot n & 1 was last read by tile n's own loads, and each
      // wave touches only its own entries of the ring and the table
      if (left >= 3) prep(n + 2, nx);
      // every wave's records of tile n have landed (each waited for its own
      // above) and its P, scales and maxima are written
      __syncthreads();

      // ---- tile max of head t over all waves (lane group g reads waves 2g, 2g+1);
      // move the reference if it grew by more than kTau
      {
        const v2f mg = *LDSP(v2f, mx + 4 * (8 * t + 2 * g));
        const float M = xor_max(fmax_(mg.x, mg.y));
        if (__builtin_amdgcn_ballot_w64(M > m_ref + kTau)) {  // the same decision in every wave
          const float m_new = fmax_(m_ref, M);
          const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
          if (__builtin_amdgcn_ballot_w64(m_ref != -INFINITY)) {  // O and l are still zero otherwise
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) O[i] *= alpha;
          }
          m_ref = m_new;
          write_p(m_ref == -INFINITY ? 0.0f : m_ref);
          __syncthreads();
        }
      }

      // ---- PV: O^T[d, h] += V^T[d, tok] P'^T[tok, h] over the tile's 128 tokens;
      // l sums the same f16 P (so numerator and denominator share the rounding)
      // K-step k's reads are issued before K-step k-1's conversions and MFMAs,
      // so one K-step's LDS latency hides behind the previous one's work.
      const uint32_t vaddr = lat + pv_off;
      v8h pr[2], sr[2];
      v2i vr[2][4];
      auto pv_load = [&](int k) __attribute__((always_inline)) {
        const int tok = 32 * k + 8 * g;
        pr[k & 1] = *LDSP(v8h, px + kPRow * t + 2 * tok);
        sr[k & 1] = *LDSP(v8h, sx + kPRow * (w >> 1) + 2 * tok);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          vr[k & 1][dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDSP(v2i, vaddr + 16 * kPair * k + 16 * dt));
      };
      pv_load(0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (k < 3) pv_load(k + 1);
        __builtin_amdgcn_sched_barrier(0);
        const v8h pk = pr[k & 1];
        const v8h pb = pk * sr[k & 1];
        l_run = __builtin_amdgcn_fdot2(v2h{pk[0], pk[1]}, ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2(v2h{pk[2], pk[3]}, ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2(v2h{pk[4], pk[5]}, ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2(v2h{pk[6], pk[7]}, ones, l_run, false);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cvt8_f16(vr[k & 1][dt]), pb, O[dt], 0, 0, 0);
      }
      if (left == 1) return;  // the last tile: nothing reuses the stage or P

      // every wave is done with stage st, P, the scales and the maxima of tile n
      __syncthreads();

      // ---- tile n+2 into stage st and this side set, then index tile n+5
      if (left >= 3) issue_next(nx, st, sd);
      if (left >= 6) {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // ring slot n+1 was read (fill_table) before its reload lands
        issue_idx(n + 5);
      }
    };

    for (int n = t0; n < t1; n += 2) {
      tile(n, 0, sA);
      if (n + 1 < t1) tile(n + 1, 1, sB);
    }
    bool pref_n = false;
    if (MULTI && has_n) {
      // every load of this unit and the next unit's descriptor have landed (the
      // last tile waited for all of them): queue the next unit's first index
      // tiles, which land during this unit's epilogue
      wait_vm_all();
      const int beg_n = __builtin_amdgcn_readlane(ud_n, 1);
      const int tiles_n = __builtin_amdgcn_readlane(ud_n, 3);
      const int ct_n = (tiles_n + S - 1) / S;
      const int t0_n = min(chunk_n * ct_n, tiles_n);
      pref_n = t0_n < min(t0_n + ct_n, tiles_n);
      if (pref_n) {
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this unit's reads of the ring are done before it is refilled
        issue_idx_at(beg_n, t0_n);
        issue_idx_at(beg_n, t0_n + 1);
        issue_idx_at(beg_n, t0_n + 2);
      }
    } else {
      wait_vm_all();  // no DMA may still target LDS when the block ends
    }

    // ---- epilogue: head t's sum over all tokens, then this wave's 64 dims
    // (split: a partial without the sink, which the combine folds in)
    l_run = xor_sum(l_run);
    const Norm nm = finish_norm(l_run, m_ref, (split || !h_ok) ? -INFINITY : sink_log2(SMLA_P(sink), h));
    const float inv = nm.scale;
    const float l2 = nm.lse2;
    if (w == 0 && g == 0 && h_ok) {
      if (split) SMLA_P(part_lse)[(int64_t)unit * H + h] = l2;
      else if (SMLA_P(lse)) SMLA_P(lse)[(int64_t)row * H + h] = l2 * kLn2;
    }
    if (split) {
      if (h_ok) st_part16(SMLA_P(part_o) + ((int64_t)unit * H + h) * kLat + 64 * w, g, O, inv);
    } else {
      // bf16 rows staged in this wave's part of the q area (idle after the
      // prologue), then read back 8 lanes per head, so that each store
      // instruction writes eight heads' 128 contiguous bytes (the wave's own
      // LDS writes, which LDS performs in order)
      const uint32_t ob = base + kQOff + w * (16 * kOutPitch);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) *LDSP(v2i, ob + kOutPitch * t + 2 * (16 * dt + 4 * g)) = pack_bf16x4(O[dt] * inv);
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int hh = 8 * i + (lane >> 3);
        const v4i v = *LDSP(v4i, ob + kOutPitch * hh + 16 * (lane & 7));
        if (hh < H) *(v4i*)(SMLA_P(out) + row * SMLA_P(o_st) + hh * SMLA_P(o_sh) + 64 * w + 8 * (lane & 7)) = v;
      }
    }
    if (!MULTI || !has_n) return;
    // every wave is past this unit (its stages, P buffers and the q area) before
    // the next unit's loads land there
    __syncthreads();
    rank = rank_n;
    chunk = chunk_n;
    have_ud = true;
    pref = pref_n;
  }  // units
#undef SMLA_P
}

// ---------------------------------------------------------------- combine

// LSE merge of a split row's chunks (K2-back page, stage_combine):
// M = max(max_c lse2_c, sink2), w_c = 2^(lse2_c - M),
// out = sum w_c o_c / (sum w_c + 2^(sink2 - M)); the sink (-inf when absent)
// is one more key whose value is 0.
// All chunk loads are issued before any is used: they are unconditional
// (chunk slots past S re-read chunk 0 and are ignored), and the f16 partials
// are converted only after the last load.
template <int SMAX>
__device__ __forceinline__ void combine_row(const float* __restrict__ part_lse, const uint16_t* __restrict__ part_o,
                                            int H, int S, const CombineParams& p, int row, int h) {
  const int64_t u0 = (int64_t)row * S;
  float lc[SMAX];
  v2i raw[SMAX];
#pragma unroll
  for (int c = 0; c < SMAX; ++c) {
    const int64_t u = u0 + (c < S ? c : 0);
    lc[c] = part_lse[u * H + h];
    raw[c] = *(const v2i*)(part_o + (u * H + h) * kLat + 4 * threadIdx.x);
  }
  const float sink2 = p.sink ? p.sink[h] * 1.4426950408889634f : -INFINITY;
  float M = sink2;
#pragma unroll
  for (int c = 0; c < SMAX; ++c)
    if (c < S) M = fmax_(M, lc[c]);
  v4f acc = v4f{0, 0, 0, 0};
  float L = 0.0f;
  if (M != -INFINITY) {
    L = __builtin_amdgcn_exp2f(sink2 - M);
#pragma unroll
    for (int c = 0; c < SMAX; ++c) {
      if (c < S && lc[c] != -INFINITY) {  // an empty chunk's o_c was never written
        const float w = __builtin_amdgcn_exp2f(lc[c] - M);
        L += w;
        acc += w * half4_to_f32(raw[c]);
      }
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const v4f o = acc * inv;
  *(v2i*)(p.out + row * p.o_st + h * p.o_sh + part_dim(4 * threadIdx.x)) = pack_bf16x4(o);
  if (threadIdx.x == 0 && p.lse)
    p.lse[(int64_t)row * p.H + h] = L > 0.0f ? (M + __builtin_log2f(L)) * kLn2 : -INFINITY;
}

// The partials, the row order and the sizes come as separate leading
// arguments, preloaded into SGPRs at wave launch: the partial loads do not
// wait for a scalar load of the parameter block.
__global__ __launch_bounds__(128) void smla_combine_kernel(
    const float* __restrict__ part_lse, const uint16_t* __restrict__ part_o, const int32_t* __restrict__ order,
    int32_t T, int32_t H, int32_t S, CombineParams p) {
  int rank, h;
  xcd_unit(H, rank, h);
  if (rank >= T) return;
  const int row = order ? order[rank] : rank;
  if (S <= 4) combine_row<4>(part_lse, part_o, H, S, p, row, h);
  else if (S <= 8) combine_row<8>(part_lse, part_o, H, S, p, row, h);
  else if (S <= 16) combine_row<16>(part_lse, part_o, H, S, p, row, h);
  else combine_row<32>(part_lse, part_o, H, S, p, row, h);
}

// ---------------------------------------------------------------- decode hook

// One wave per record: the latent exactly as the QK stage sees it (e4m3 ->
// bf16 by v_cvt_scalef32_pk_bf16_fp8 with the record scale; that conversion
// uses only the scale's exponent field, so a zero scale acts as 2^-127 and a
// non-power-of-two scale as its power-of-two part).  For a valid scale (a
// positive normal power of two) it is cross-checked against the PV stage's
// conversion (e4m3 -> f16 unscaled, times the scale in f32); a disagreement
// turns the value into NaN.  Rope: bf16 -> f32.
__global__ __launch_bounds__(64) void smla_decode_rows_kernel(const uint8_t* kv, int64_t n_kv,
                                                               const int32_t* rows, int64_t n,
                                                               float* out) {
  const int64_t i = blockIdx.x;
  const int lane = threadIdx.x;
  float* o = out + i * 576;
  const int r = rows[i];
  if (r < 0 || r >= n_kv) {
    for (int d = lane; d < 576; d += 64) o[d] = __builtin_nanf("");
    return;
  }
  const uint8_t* rec = kv + (int64_t)r * kRecordBytes;
  const v2i w = *(const v2i*)(rec + 8 * lane);  // codes 8*lane .. 8*lane+7
  const float sc = *(const float*)(rec + kScaleOff + 4 * ((8 * lane) / 128));
  const uint32_t sbits = __builtin_bit_cast(uint32_t, sc);
  const uint32_t sexp = (sbits >> 23) & 0xFF;
  const bool valid_scale = (sbits & 0x807FFFFFu) == 0 && sexp >= 1 && sexp <= 254;
  v2bf a0, a1, a2, a3;
  cvt4_bf16(w.x, sc, a0, a1);
  cvt4_bf16(w.y, sc, a2, a3);
  const __bf16 vb[8] = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
  const v8h vh = cvt8_f16(w);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float v = (float)vb[k];
    const float viaf16 = (float)vh[k] * sc;
    const bool agree = (v == viaf16) || (v != v && viaf16 != viaf16);
    o[8 * lane + k] = (!valid_scale || agree) ? v : __builtin_nanf("");
  }
  const uint16_t rb = *(const uint16_t*)(rec + kRopeOff + 2 * lane);
  o[kLat + lane] = __builtin_bit_cast(float, (uint32_t)rb << 16);
}

// ---------------------------------------------------------------- cache writer

// Writes token i's record at kv[slots[i]] by the fp8_ds_mla writer rule (FlyDSL
// page, module docstring, "Preconditions the host cannot check"): per 128
// latent values scale = pow2ceil(max(amax, 1e-4) / 448), an f32 power of two;
// latent codes = e4m3(x / scale), rounded to nearest even; rope copied as bf16.
// One wave per token: lane l holds latent values 8l .. 8l+7, so scale block b
// is lanes 16b .. 16b+15.
__global__ __launch_bounds__(256) void smla_cache_write_kernel(CacheWriteParams p) {
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= p.n) return;
  const int lane = threadIdx.x & 63;
  const v4i raw = *(const v4i*)(p.latent + i * p.latent_st + 8 * lane);  // 8 bf16
  const v2i rp = lane < 16 ? *(const v2i*)(p.rope + i * p.rope_st + 4 * lane) : v2i{0, 0};
  const int64_t slot = p.slots[i];
  if (slot < 0 || slot >= p.n_kv) return;  // padding tokens; out-of-range slots are never written
  uint8_t* rec = p.kv + slot * kRecordBytes;

  float x[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __builtin_bit_cast(float, (uint32_t)raw[k] << 16);
    x[2 * k + 1] = __builtin_bit_cast(float, (uint32_t)raw[k] & 0xFFFF0000u);
  }
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmax_(amax, __builtin_fabsf(x[k]));
  // max over the 16 lanes of the scale block, by DPP: quad_perm xor 1 and
  // xor 2 (quads), row_half_mirror (lanes i <-> 7 - i: pairs the quads of a
  // half row), row_mirror (i <-> 15 - i: pairs the half rows)
#define SMLA_DPP_MAX(ctrl) \
  amax = fmax_(amax, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, amax), ctrl, 0xF, 0xF, false)))
  SMLA_DPP_MAX(0xB1);
  SMLA_DPP_MAX(0x4E);
  SMLA_DPP_MAX(0x141);
  SMLA_DPP_MAX(0x140);
#undef SMLA_DPP_MAX
  // pow2ceil of v = max(amax, 1e-4) / 448 (a positive normal f32): v itself if
  // its mantissa is zero, else the next power of two.  The f32 quotient is a
  // power of two exactly when the exact one is (amax has 8 significant bits),
  // so the result is the exact rule's.
  const float v = fmax_(amax, 1e-4f) / 448.0f;
  const uint32_t vb = __builtin_bit_cast(uint32_t, v);
  const uint32_t sb = (vb & 0x007FFFFFu) ? (vb & 0x7F800000u) + 0x00800000u : vb;
  const float scale = __builtin_bit_cast(float, sb);
  const float inv = __builtin_bit_cast(float, 0x7F000000u - sb);  // 1 / scale, exact
  int w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0] * inv, x[1] * inv, w0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2] * inv, x[3] * inv, w0, true);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4] * inv, x[5] * inv, w1, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6] * inv, x[7] * inv, w1, true);
  *(v2i*)(rec + 8 * lane) = v2i{w0, w1};
  if ((lane & 15) == 0) *(float*)(rec + kScaleOff + 4 * (lane >> 4)) = scale;
  if (lane < 16) *(v2i*)(rec + kRopeOff + 8 * lane) = rp;
}

// ---------------------------------------------------------------- launchers

hipError_t zero_record_address(const uint8_t** out) {
  void* ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_zero_record));
  *out = (const uint8_t*)ptr;
  return e;
}

hipError_t launch_plan(const PlanParams& p, bool sort, Events ev, hipStream_t s) {
  if (p.has_invalid) {
    hipExtLaunchKernelGGL(smla_plan_scan_kernel, dim3(p.T), dim3(256), 0, s, ev.start,
                          sort ? nullptr : ev.stop, 0, p.indptr, p.indices, p.idx_bytes, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (sort) {
    hipExtLaunchKernelGGL(smla_plan_sort_kernel, dim3(1), dim3(1024), 0, s,
                          p.has_invalid ? nullptr : ev.start, ev.stop, 0, p.row_tiles, p.indptr, p.T,
                          p.has_invalid, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_fwd(const FwdParams& p, Events ev, hipStream_t s) {
  switch (head_tiles(p.H)) {
    case 1: {
      const int64_t blocks = fwd_grid(p.T, p.S, p.order == nullptr);
      // with the plan and more units than the persistent grid (p.persist
      // blocks, one per CU) but at most two per block, the persistent kernel;
      // otherwise one unit per block (with more units per CU the hardware's
      // dispatch of blocks as CUs free up balances ragged rows better)
      if (p.persist > 0 && p.desc != nullptr && blocks > p.persist && blocks <= 2 * (int64_t)p.persist)
        hipExtLaunchKernelGGL(smla_fwd16_kernel<true>, dim3((unsigned)p.persist), dim3(n16::kThreads), 0, s,
                              ev.start, ev.stop, 0, p.indptr, p.indices, p.q, p.desc, p.T, p.S, p.idx_bytes, p.stride, p);
      else
        hipExtLaunchKernelGGL(smla_fwd16_kernel<false>, dim3((unsigned)blocks), dim3(n16::kThreads), 0, s,
                              ev.start, ev.stop, 0, p.indptr, p.indices, p.q, p.desc, p.T, p.S, p.idx_bytes, p.stride, p);
      return hipGetLastError();
    }
    default: return launch_fwd_wide(p, ev, s);
  }
}

hipError_t launch_combine(const CombineParams& p, Events ev, hipStream_t s) {
  const int64_t blocks = xcd_grid(p.T, p.H);
  hipExtLaunchKernelGGL(smla_combine_kernel, dim3((unsigned)blocks), dim3(128), 0, s, ev.start, ev.stop, 0,
                        p.part_lse, p.part_o, p.order, p.T, p.H, p.S, p);
  return hipGetLastError();
}

hipError_t launch_cache_write(const CacheWriteParams& p, Events ev, hipStream_t s) {
  const int64_t blocks = (p.n + 3) / 4;
  hipExtLaunchKernelGGL(smla_cache_write_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ev.start, ev.stop, 0, p);
  return hipGetLastError();
}

hipError_t launch_decode_rows(const uint8_t* kv, int64_t n_kv, const int32_t* rows, int64_t n,
                              float* out, hipStream_t s) {
  hipLaunchKernelGGL(smla_decode_rows_kernel, dim3((unsigned)n), dim3(64), 0, s, kv, n_kv, rows, n, out);
  return hipGetLastError();
}

}  // namespace smla
