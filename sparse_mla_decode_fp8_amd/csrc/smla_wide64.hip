// Wide-head forward for 33 <= H <= 128 heads (up to 64 heads per unit; above
// 64 a row's heads form groups of 64, each its own unit): the prefill and
// wide decode shapes.  Same method as the other forward kernels (vLLM API
// page "vllm.models.kimi_k3.amd.ops.flydsl_sparse_mla_gfx950", module
// docstring; split chunks merged as on the K2-back page, stage_combine).
//
// The eight waves of a block have two roles.  Waves w and w + 4 of a block
// run on the same SIMD, so every SIMD holds one wave of each role, and the
// conversion-heavy score work of one overlaps the MFMA-heavy P.V work of the
// other instead of both waves of a SIMD doing the same phase at once.
//   QK waves 0..3: wave (h, k) = (w & 1, w >> 1) computes the dim-half-h
//       part of the scores (latent dims 256h .. 256h+255 and rope dims
//       32h .. 32h+31) of all 64 heads against tokens 16k .. 16k+15 of each
//       32-token tile, so each K element is converted once per tile.  The
//       wave sends the other half's head tiles to it through LDS and, one
//       step later, adds the half it receives and runs the softmax of heads
//       32h .. 32h+31.  The two token halves are two softmax streams: each
//       wave keeps its own running reference and sum per head, writes P
//       relative to its reference and publishes the reference.  References
//       are integers (log2 units), so every factor between them is an exact
//       power of two.
//   PV waves 4..7: wave 4 + j owns dims 128j .. 128j+127, one scale block,
//       for all 64 heads, so the block's per-token V scale folds into P; it
//       keeps O relative to the larger of the two streams' references,
//       scales each stream's P to it, and accumulates O over the tile whose
//       softmax ran one step before.  These waves also run the gather: index
//       tiles into an LDS ring and the records (latent rows, scales and
//       rope) of 8 tokens per tile.
// One barrier per step: at step s the QK waves score tile s and run the
// softmax of tile s - 1 while the PV waves work on tile s - 2 and queue the
// records of tile s + 3 (three tiles of records in flight, six LDS stages).
// Halves of scores, P, the V scales and the references are double-buffered
// by tile parity.  The two streams are merged like two chunks of a split row
// (K2-back page, stage_combine).

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "smla_device.h"

namespace smla {
namespace w64 {

typedef uint64_t v2u64 __attribute__((ext_vector_type(2)));
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kHeads = 64;
constexpr int kTile = 32;                       // tokens per step
constexpr int kAhead = 3;                       // tiles of records queued ahead of the QK tile
constexpr int kStages = kAhead + 3;             // LDS record stages
constexpr int kRing = 16;                       // index ring slots (tiles), >= 2 kAhead + 1
constexpr int kPair = 2 * kLat + 16;            // two latent rows + 16-B pad
constexpr int kLatStage = (kTile / 2) * kPair;  // 16,640 B
constexpr int kSideStage = kTile * kSideTok;    // 4,608 B
constexpr int kPitch = 96;                      // P and scale rows: 32 f16 + pad (no 128-bit read conflicts)
// Vector-memory instructions a PV wave issues per tile: 4 latent DMAs (token
// pairs) and 2 side DMAs (72 chunks of 16 B); one index DMA besides.
constexpr int kTileVm = 6;
constexpr int kQLoads = 18;                     // q loads per lane (16 latent + 2 rope)
constexpr int kOutPitch = 2 * 128 + 16;         // epilogue staging row: 128 bf16 dims + pad

constexpr int kLatOff = 0;
constexpr int kSideOff = kLatOff + kStages * kLatStage;
constexpr int kPxOff = kSideOff + kStages * kSideStage;  // P f16 [buf 2][head 64][token], pitch kPitch
constexpr int kPxBuf = kHeads * kPitch;
constexpr int kSxOff = kPxOff + 2 * kPxBuf;               // V scales f16 [buf 2][block 4][token]
constexpr int kSxBuf = 4 * kPitch;
constexpr int kMxOff = kSxOff + 2 * kSxBuf;               // stream references f32 [buf 2][stream 2][head t 16][tile 4]
constexpr int kMxBuf = 2 * kHeads * 4;
constexpr int kSpOff = kMxOff + 2 * kMxBuf;               // halves of scores v4f [buf 2][stream 2][head tile 4][lane 64]
constexpr int kSpBuf = 2 * 4 * 64 * 16;
constexpr int kRingOff = kSpOff + 2 * kSpBuf;             // index entries [slot][32]
constexpr int kTabOff = kRingOff + kRing * kTile * 4;     // record addresses [PV wave][8]
constexpr int kKeyOff = kTabOff + 4 * 64;                 // key masks u32 [slot]: bit i = token i is a key
constexpr int kRedOff = kKeyOff + kRing * 4;              // unit_tiles' reduction; later {l, m} per head and stream
constexpr int kBytes = kRedOff + kHeads * 16;
// q exchange before the first tile (18 KB per score wave): waves 0, 1 in record
// stages 3.. of the latent area, waves 2, 3 from record stage 3 of the side
// area on (over P, scales, references and halves of scores); none of these is
// written before the first tile's step.
constexpr int kQxBytes = 18 * 64 * 16;
constexpr int kQxA = kLatOff + 3 * kLatStage;
constexpr int kQxB = kSideOff + 3 * kSideStage;
static_assert(kQxA + 2 * kQxBytes <= kSideOff && kQxB + 2 * kQxBytes <= kRingOff, "q exchange areas");
static_assert(kBytes <= 160 * 1024, "LDS budget");
static_assert(4 * kHeads * kOutPitch <= kStages * kLatStage, "epilogue staging fits the latent stages");
static_assert(kStages >= kAhead + 3 && kRing >= 2 * kAhead + 1, "pipeline depth");

// vmcnt <= n for a wave-uniform n in [0, 24]
__device__ __forceinline__ void wait_vm_n(int n) {
  switch (n) {
#define SMLA_W(k) case k: wait_vm<k>(); break;
    SMLA_W(0) SMLA_W(1) SMLA_W(2) SMLA_W(3) SMLA_W(4) SMLA_W(5) SMLA_W(6) SMLA_W(7) SMLA_W(8)
    SMLA_W(9) SMLA_W(10) SMLA_W(11) SMLA_W(12) SMLA_W(13) SMLA_W(14) SMLA_W(15) SMLA_W(16)
    SMLA_W(17) SMLA_W(18) SMLA_W(19) SMLA_W(20) SMLA_W(21) SMLA_W(22) SMLA_W(23)
#undef SMLA_W
    default: wait_vm<24>(); break;
  }
}

__device__ __forceinline__ uint32_t row_off(int tau) { return (tau >> 1) * kPair + (tau & 1) * kLat; }

}  // namespace w64

// PAGED: the keys live in paged pools (KeyMode, key_addr); otherwise in one
// contiguous cache (entries >= 0 are keys), compiled without the pool logic.
// MULTI: a persistent grid (a multiple of 8 blocks, one per CU at most): block
// b runs one virtual block of the one-unit-per-block grid in each round k, in
// turn: k * grid + b in even rounds and k * grid + b' in odd ones, b' being b
// mirrored among the blocks of its XCD.  In the plan's longest-first order a
// block's units then pair long with short, and each runs on the XCD the plain
// grid would use.  At a unit's last steps the score waves
// load their q of the next unit and the P.V waves queue its first index tiles,
// so the next unit starts with both at hand.  It runs with the plan
// only (units from the plan's descriptors).
template <bool PAGED, bool MULTI>
__global__ __launch_bounds__(w64::kThreads, 1) void smla_fwdw64_kernel(FwdParams p) {
  using namespace w64;
  __shared__ __attribute__((aligned(1024))) uint8_t s_lds[kBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 15;
  const int g = lane >> 4;

  const int per_row = p.S * p.hg;
  int vb = 0;  // (persistent) the round: which of the block's units this is
  int rank, sub;
  // all chunks and head groups of a row on one XCD: the row's q is fetched
  // into that XCD's L2 once
  xcd_unit_at(blockIdx.x, per_row, rank, sub);
  if (!MULTI && rank >= p.T) return;

  const uint32_t base = lds_addr(s_lds);
  const __amdgpu_buffer_rsrc_t irs = idx_rsrc(p.indices, p.idx_bytes);
  auto ring_at = [&](int n) -> uint32_t { return base + kRingOff + (n & (kRing - 1)) * kTile * 4; };
  // I: index DMA of PV wave j's 8 entries of tile n of the slice starting at
  // b (bounded reads: positions past nnz read 0; positions past the row are
  // masked where they are used).
  auto issue_idx_at = [&](int b, int n) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(ring_at(n) + 32 * (w - 4));
    if (lane < 8) buf_dma4(irs, (uint32_t)(b + n * kTile + 8 * (w - 4) + lane) * 4u, dst);
  };
  // Without a plan and with a uniform slice stride, the PV waves guess the
  // slice start (rank * stride) and queue the unit's first index tiles before
  // indptr arrives; they queue them again from the real start if the guess
  // was wrong.
  const int stride = MULTI ? 0 : p.stride;
  const int ct_g = ((stride + kTile - 1) / kTile + p.S - 1) / p.S;
  const int t0_g = min((sub % p.S) * ct_g, (stride + kTile - 1) / kTile);
  const int t1_g = min(t0_g + ct_g, (stride + kTile - 1) / kTile);
  const int beg_g = rank * stride;
  const bool spec = stride > 0 && w >= 4;
  if (spec) {
#pragma unroll
    for (int k = 0; k < kAhead; ++k)
      if (t0_g + k < t1_g) issue_idx_at(beg_g, t0_g + k);
  }
  const bool split = p.S > 1;
  const int H = p.H;
  // (persistent) kernel arguments read at a unit's start and end come through
  // a pointer the compiler cannot see through, so they are loaded where they
  // are used instead of being held in registers through every unit's steps
  typedef const __attribute__((address_space(4))) FwdParams* KArgs;
  auto args = [&]() -> KArgs {
    KArgs a = (KArgs)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(a));
    return a;
  };
#define SMLA_ARG(a, f) (MULTI ? (a)->f : p.f)
  // a unit: its row, head group, slice and tile range
  struct Unit {
    int row, chunk, h0, beg, len, t0, t1;
  };
  auto unit_at = [&](int r, int sb, Unit& uu) {
    const KArgs ka = args();
    const int S = SMLA_ARG(ka, S);
    const int32_t* const desc = SMLA_ARG(ka, desc);
    const int32_t* const indptr = SMLA_ARG(ka, indptr);
    uu.chunk = sb % S;
    uu.h0 = kHeads * (sb / S);  // first head of the unit's head group
    int tiles;
    if (MULTI || desc) {  // the plan's unit of rank r in one load
      const v4i d = *(const v4i*)(desc + 4 * r);
      uu.row = d.x;
      uu.beg = d.y;
      uu.len = d.z;
      tiles = d.w;
    } else {
      uu.row = r;
      uu.beg = indptr[r];
      uu.len = max(indptr[r + 1] - uu.beg, 0);
      tiles = unit_tiles<kThreads>(p, r, uu.beg, uu.len, kTile, (int*)(s_lds + kRedOff));
    }
    const int ct = (tiles + S - 1) / S;
    uu.t0 = min(uu.chunk * ct, tiles);
    uu.t1 = min(uu.t0 + ct, tiles);
  };
  // (persistent) the block's first unit after round k that holds a row
  auto next_unit = [&](int& k, Unit& uu) -> bool {
    const KArgs ka = args();
    const int T = SMLA_ARG(ka, T), pr = SMLA_ARG(ka, S) * SMLA_ARG(ka, hg);
    const int nvb = 8 * ((T + 7) / 8) * pr;
    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    const int mirror = (b & 7) + 8 * (G / 8 - 1 - (b >> 3));
    for (++k; k * G < nvb; ++k) {
      const int v = k * G + ((k & 1) ? mirror : b);
      if (v >= nvb) continue;
      int r, sb;
      xcd_unit_at(v, pr, r, sb);
      if (r < T) {
        unit_at(r, sb, uu);
        return true;
      }
    }
    return false;
  };
  Unit u;
  if (rank < p.T) unit_at(rank, sub, u);
  else if (!next_unit(vb, u)) return;

  const uint32_t px0 = base + kPxOff;
  const uint32_t sx0 = base + kSxOff;
  const uint32_t mx0 = base + kMxOff;
  const uint32_t keys = base + kKeyOff;
  const uint32_t lm = base + kRedOff;  // {l, m} of head h, stream k at lm + 16h + 8k (epilogue)
  auto lat_at = [&](int st) -> uint32_t { return base + kLatOff + st * kLatStage; };
  auto side_at = [&](int st) -> uint32_t { return base + kSideOff + st * kSideStage; };

  // (both roles) a unit with nothing to attend: zero output and the sink's
  // lse, or an empty partial
  auto empty_unit = [&](const Unit& uu) {
    const int Hu = min(H - uu.h0, kHeads);
    const int64_t uid = (int64_t)uu.row * p.S + uu.chunk;
    if (spec) wait_vm<0>();  // the guessed index tiles land before the block ends
    const KArgs ka = args();
    if (split) {
      float* const part_lse = SMLA_ARG(ka, part_lse);
      for (int hh = uu.h0 + tid; hh < uu.h0 + Hu; hh += kThreads) part_lse[uid * H + hh] = -INFINITY;
    } else {
      uint16_t* const out = SMLA_ARG(ka, out);
      const int64_t o_st = SMLA_ARG(ka, o_st), o_sh = SMLA_ARG(ka, o_sh);
      for (int e = tid; e < Hu * (kLat / 8); e += kThreads) {
        const int hh = uu.h0 + e / (kLat / 8), d = (e % (kLat / 8)) * 8;
        *(v4i*)(out + uu.row * o_st + hh * o_sh + d) = v4i{0, 0, 0, 0};
      }
      float* const lse = SMLA_ARG(ka, lse);
      const float* const sink = SMLA_ARG(ka, sink);
      if (lse)
        for (int hh = uu.h0 + tid; hh < uu.h0 + Hu; hh += kThreads)
          lse[(int64_t)uu.row * H + hh] = sink ? sink[hh] : -INFINITY;
    }
  };
  // Each role runs the same units in the same order and meets the same
  // barriers.  Each has a loop of its own, so that what it carries from one
  // unit to the next (the score waves' q pair) takes no registers in the other.
  if (w < 4) {
    bool pref = false;  // (persistent) this unit's own q pair and first index tiles were queued by the unit before
    v4i qn[2][9];  // this wave's own q pair of the unit (queued by the unit before, or at its start)
    for (;;) {
      // (persistent) lane-derived values are formed anew in each unit, from an
      // opaque copy of the lane index, instead of being held across units
      int lane_u = lane;
      if (MULTI) asm volatile("" : "+v"(lane_u));
      const int lane = lane_u, t = lane & 15, g = lane >> 4;
      const int row = u.row, chunk = u.chunk, h0 = u.h0, beg = u.beg, len = u.len, t0 = u.t0, t1 = u.t1;
      const int unit = row * p.S + chunk;
      const int Hl = min(H - h0, kHeads);  // heads of this group
      if (t0 >= t1) {
        empty_unit(u);
        if (!MULTI || !next_unit(vb, u)) return;
        pref = false;
        continue;
      }
      // (persistent) the unit to come; both roles look it up at the unit's
      // last step, not holding it in registers through the steps
      int vbn = vb;
      Unit un{};
      bool has_next = false, pref_next = false;
      auto find_next = [&]() {
        has_next = next_unit(vbn, un);
        pref_next = has_next && un.t0 < un.t1;
        asm volatile("" ::"s"(un.row), "s"(un.h0), "s"(un.beg), "s"(un.len), "s"(un.t0), "s"(un.t1));
      };
      // ================================================================ QK waves
      const int h = w & 1;    // dim half of the scores; softmax of heads 32h .. 32h+31
      const int kq = w >> 1;  // token half (stream): tokens 16kq .. 16kq+15 of a tile
      // q of head tile (2h + v) & 3 (heads 16((2h + v) & 3) + t, lane (t, g)),
      // so tiles v = 0, 1 are this wave's softmax heads and v = 2, 3 the other
      // wave's: latent K-step 2m / 2m+1 (m = 0..3) = dims 256h + 64m + 16g +
      // [0..7] / [8..15], rope K-step = dims 512 + 32h + 8g + [0..7].  Heads >= H
      // load head 0 (every lane issues the same loads) and are zeroed.
      // The two waves of a dim half need the same q: wave (h, kq) loads head
      // tiles v = 2kq, 2kq+1 (18 loads per lane), publishes them in LDS and,
      // after a barrier, reads the other two that wave (h, 1 - kq) loaded.
      v8bf qlat[4][8], qrope[4];
      auto qx_at = [&](int wave) -> uint32_t { return base + (wave < 2 ? kQxA : kQxB) + (wave & 1) * kQxBytes; };
      auto take = [&](int v, const v4i (&qr)[9]) {
        const bool hq_ok = 16 * ((2 * h + v) & 3) + t < Hl;
#pragma unroll
        for (int k = 0; k < 8; ++k) qlat[v][k] = __builtin_bit_cast(v8bf, hq_ok ? qr[k] : v4i{0, 0, 0, 0});
        qrope[v] = __builtin_bit_cast(v8bf, hq_ok ? qr[8] : v4i{0, 0, 0, 0});
      };
      // this wave's own head tiles v = 2kq, 2kq+1 of unit uu (18 loads per lane into qr)
      auto issue_pair = [&](const Unit& uu, v4i (&qr)[2][9]) {
        const int Hu = min(H - uu.h0, kHeads);
        const KArgs ka = args();
        const uint16_t* const qb = SMLA_ARG(ka, q) + uu.row * SMLA_ARG(ka, q_st);
        const int64_t q_sh = SMLA_ARG(ka, q_sh);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int hq = 16 * ((2 * h + 2 * kq + i) & 3) + t;
          const uint64_t qa = (uint64_t)(uintptr_t)(qb + (int64_t)(uu.h0 + (hq < Hu ? hq : 0)) * q_sh);
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            gload16(qr[i][2 * m], qa + 2 * (256 * h + 64 * m + 16 * g));
            gload16(qr[i][2 * m + 1], qa + 2 * (256 * h + 64 * m + 16 * g + 8));
          }
          gload16(qr[i][8], qa + 2 * (kLat + 32 * h + 8 * g));
        }
      };
      // the own pair, once landed: published in LDS for the other wave of the
      // dim half and taken as head tiles v0, v0 + 1 (v0 = 2kq)
      auto publish_pair = [&](auto V0, v4i (&qr)[2][9]) {
        constexpr int v0 = decltype(V0)::value;
        wait_vm<0>();
        const uint32_t dst = qx_at(w) + 16 * lane;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int k = 0; k < 9; ++k) {
            asm volatile("" : "+v"(qr[i][k]));
            *LDSP(v4i, dst + (9 * i + k) * 1024) = qr[i][k];
          }
        take(v0, qr[0]);
        take(v0 + 1, qr[1]);
      };
      auto read_pair = [&](auto V0) {
        constexpr int v0 = decltype(V0)::value;
        const uint32_t src = qx_at(w ^ 2) + 16 * lane;
        v4i qr[2][9];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int k = 0; k < 9; ++k) qr[i][k] = *LDSP(v4i, src + (9 * i + k) * 1024);
        take(v0, qr[0]);
        take(v0 + 1, qr[1]);
      };
      // wave (h, kq) loads tiles 2(h ^ kq), 2(h ^ kq) + 1: own tiles (v = 0, 1) when kq = 0
      // (persistent: already queued at the previous unit's last step)
      if (MULTI) {
        // (each wave's two branches below write all four head tiles between
        // them; defined here first, the previous unit's q is not carried over)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
#pragma unroll
          for (int k = 0; k < 8; ++k) qlat[v][k] = v8bf{};
          qrope[v] = v8bf{};
        }
      }
      if (!pref) issue_pair(u, qn);
      if (kq == 0) publish_pair(std::integral_constant<int, 0>{}, qn);
      else publish_pair(std::integral_constant<int, 2>{}, qn);
      __syncthreads();
      if (kq == 0) read_pair(std::integral_constant<int, 2>{});
      else read_pair(std::integral_constant<int, 0>{});

      float m_ref[2] = {-INFINITY, -INFINITY};  // head 32h + 16u + t, this stream: reference (log2 units, integer)
      float eo[2] = {kShift, kShift};           // kShift - m_ref (kShift while m_ref is -inf): P = 2^(x + eo)
      float l_run[2] = {0.0f, 0.0f};            // this lane's part of the stream's sum of P
      v4f own[2];                               // this dim half's scores of the previous tile, heads 32h + 16u + t
      const v2h ones = v2h{(_Float16)1.0f, (_Float16)1.0f};
      const int tok = 16 * kq + t;  // the token whose K row this lane feeds
      const uint32_t qk_row = row_off(tok) + 16 * g + 256 * h;
      const uint32_t qk_a = qk_row + ((t & 1) ? 128u : 0u);
      const uint32_t qk_b = qk_row - ((t & 1) ? 128u : 0u);
      // halves of scores: [buffer 2][stream 2][head tile 4][lane] v4f; each
      // wave writes the head tiles of the other dim half's wave and reads its own
      const uint32_t sp_w = base + kSpOff + 16 * (64 * (4 * kq + 2 - 2 * h) + lane);
      const uint32_t sp_r = base + kSpOff + 16 * (64 * (4 * kq + 2 * h) + lane);

      // this dim half's scores of the tile in stage st: lane (t, g) gets heads
      // 16((2h + v) & 3) + t, tokens 16kq + 4g + r; each K element is converted
      // once for all 64 heads (one accumulator chain per head tile)
      auto half_scores = [&](int st, v4f (&acc)[4]) {
        const uint32_t lat = lat_at(st);
        const uint32_t side = side_at(st) + kSideTok * tok;
        const v8bf rp = __builtin_bit_cast(v8bf, *LDSP(v4i, side + 16 + 64 * h + 16 * g));
        const v2f ksc = *LDSP(v2f, side + 8 * h);  // scales of blocks 2h, 2h+1
        v4i kr[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) kr[m] = *LDSP(v4i, lat + ((m & 2) ? qk_b : qk_a) + 64 * m);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rp, qrope[v], v4f{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float sc = ksc[m >> 1];
          v2bf a0, a1, a2, a3, b0, b1, b2, b3;
          cvt4_bf16(kr[m].x, sc, a0, a1);
          cvt4_bf16(kr[m].y, sc, a2, a3);
          cvt4_bf16(kr[m].z, sc, b0, b1);
          cvt4_bf16(kr[m].w, sc, b2, b3);
          const v8bf ka = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
          const v8bf kb = {b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qlat[v][2 * m], acc[v], 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qlat[v][2 * m + 1], acc[v], 0, 0, 0);
        }
      };
      // the other dim half's head tiles go to its wave through LDS
      auto send_half = [&](int n, const v4f (&acc)[4]) {
        const uint32_t a = sp_w + (n & 1) * kSpBuf;
        *LDSP(v4f, a) = acc[2];
        *LDSP(v4f, a + 64 * 16) = acc[3];
      };
      // softmax of tile n (stage st) for heads 32h + 16u + t: the scores are
      // this wave's half plus the other wave's; P, the references and the V
      // scales go to the buffers of tile parity n & 1
      auto softmax = [&](int n, int st) {
        const int b = n & 1;
        const uint32_t kmask = *LDSP(uint32_t, keys + 4 * (n & (kRing - 1)));
        const float vsc = *LDSP(float, side_at(st) + kSideTok * tok + 4 * g);
        const v4f o0 = *LDSP(v4f, sp_r + b * kSpBuf);
        const v4f o1 = *LDSP(v4f, sp_r + b * kSpBuf + 64 * 16);
        // V scale of block g for token tok, clamped to 2^7, as f16 (the waves
        // of dim half 0 write it)
        if (h == 0) *LDSP(_Float16, sx0 + b * kSxBuf + kPitch * g + 2 * tok) = (_Float16)__builtin_fminf(vsc, kScaleCap);
        const uint32_t kb = kmask >> (16 * kq + 4 * g);  // which of tokens 16kq + 4g + r are keys
        const float c = p.c_log2;  // > 0: the scaled max is the max of the scaled scores
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const v4f S = own[u] + (u ? o1 : o0);
          float y[4];  // the scores of keys, -inf elsewhere
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = ((kb >> r) & 1u) ? S[r] : -INFINITY;
          float tmax = fmax_(fmax_(y[0], y[1]), fmax_(y[2], y[3])) * c;
          // the head's max over this tile's half; the stream's reference
          // moves (to the max rounded up) only when the max exceeds it by
          // more than kTau.  The lanes' maxima are reduced over the head's
          // four lanes only when some lane's exceeds (a wave-wide ballot).
          if (__builtin_amdgcn_ballot_w64(tmax > m_ref[u] + kTau)) {
            tmax = xor_max(tmax);
            if (tmax > m_ref[u] + kTau) {
              const float m_new = __builtin_ceilf(tmax);
              if (m_ref[u] != -INFINITY) l_run[u] *= __builtin_amdgcn_ldexpf(1.0f, (int)__builtin_fmaxf(m_ref[u] - m_new, -200.0f));
              m_ref[u] = m_new;
              eo[u] = kShift - m_new;
            }
          }
          const int hh = 32 * h + 16 * u + t;  // head of the group
          // (the four lanes of a head write the same value)
          *LDSP(float, mx0 + b * kMxBuf + kq * (kHeads * 4) + 16 * t + 4 * (2 * h + u)) = m_ref[u];
          _Float16 ph[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ph[r] = (_Float16)__builtin_amdgcn_exp2f(__builtin_fmaf(y[r], c, eo[u]));
          l_run[u] = __builtin_amdgcn_fdot2(v2h{ph[0], ph[1]}, ones, l_run[u], false);
          l_run[u] = __builtin_amdgcn_fdot2(v2h{ph[2], ph[3]}, ones, l_run[u], false);
          *LDSP(v2i, px0 + b * kPxBuf + kPitch * hh + 2 * (16 * kq + 4 * g)) =
              __builtin_bit_cast(v2i, (v4h{ph[0], ph[1], ph[2], ph[3]}));
        }
      };

      // Step s (t0 <= s <= t1 + 1, one barrier each): this half of tile s's
      // scores, and the softmax of tile s - 1, whose other half arrived over
      // the barrier.  At the barrier of step s tile s's records have landed
      // and the PV waves are done with tile s - 3, whose P, scale and
      // reference buffers tile s - 1 takes.
      __syncthreads();
      {
        v4f acc[4];
        half_scores(0, acc);
        send_half(t0, acc);
        own[0] = acc[0];
        own[1] = acc[1];
      }
      int st = 1;  // stage of tile s
      for (int s = t0 + 1; s < t1; ++s) {
        __syncthreads();
        const int st_prev = st == 0 ? kStages - 1 : st - 1;
        v4f acc[4];
        half_scores(st, acc);
        softmax(s - 1, st_prev);
        send_half(s, acc);
        own[0] = acc[0];
        own[1] = acc[1];
        st = st == kStages - 1 ? 0 : st + 1;
      }
      __syncthreads();
      softmax(t1 - 1, st == 0 ? kStages - 1 : st - 1);
      if (MULTI) {
        // the next unit's own pair, landing during this unit's end (and qn
        // defined on both paths, so nothing holds it between units' uses)
        find_next();
        if (pref_next) issue_pair(un, qn);
        else
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int k = 0; k < 9; ++k) qn[i][k] = v4i{0, 0, 0, 0};
      }
      __syncthreads();  // step t1 + 1: the PV waves' last tile
      // each head's stream sum and reference for the PV waves' normalisation
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float l = xor_sum(l_run[u]);
        if (g == 0) *LDSP(v2f, lm + 16 * (32 * h + 16 * u + t) + 8 * kq) = v2f{l, m_ref[u]};
      }
      __syncthreads();
      if (!MULTI || !has_next) return;
      // every wave is past this unit's epilogue (staged in the record
      // stages) before the next unit's q exchange and records land there
      __syncthreads();
      vb = vbn;
      u = un;
      pref = pref_next;
    }
  } else {
    bool pref = false;  // (persistent) this unit's own q pair and first index tiles were queued by the unit before
    for (;;) {
      // (persistent) lane-derived values are formed anew in each unit, from an
      // opaque copy of the lane index, instead of being held across units
      int lane_u = lane;
      if (MULTI) asm volatile("" : "+v"(lane_u));
      const int lane = lane_u, t = lane & 15, g = lane >> 4;
      const int row = u.row, chunk = u.chunk, h0 = u.h0, beg = u.beg, len = u.len, t0 = u.t0, t1 = u.t1;
      const int unit = row * p.S + chunk;
      const int Hl = min(H - h0, kHeads);  // heads of this group
      if (t0 >= t1) {
        empty_unit(u);
        if (!MULTI || !next_unit(vb, u)) return;
        pref = false;
        continue;
      }
      // (persistent) the unit to come; both roles look it up at the unit's
      // last step, not holding it in registers through the steps
      int vbn = vb;
      Unit un{};
      bool has_next = false, pref_next = false;
      auto find_next = [&]() {
        has_next = next_unit(vbn, un);
        pref_next = has_next && un.t0 < un.t1;
        asm volatile("" ::"s"(un.row), "s"(un.h0), "s"(un.beg), "s"(un.len), "s"(un.t0), "s"(un.t1));
      };
      // ================================================================== PV waves
      const int j = w - 4;  // scale block: dims 128j .. 128j+127; gather: tokens 8j .. 8j+7
      const uint8_t* const zero = p.zero;
      const uint32_t tab = base + kTabOff + 64 * j;  // this wave's 8 record addresses

      // I: index DMA of this wave's 8 entries of tile n of the row's slice
      auto issue_idx = [&](int n) { issue_idx_at(beg, n); };
      // record addresses of this wave's 8 tokens of tile n (no key: the zero
      // record), and their bits of the tile's key mask
      auto fill_table = [&](int n) {
        bool ok = false;
        if (lane < 8) {
          const int raw = *LDSP(int, ring_at(n) + 4 * (8 * j + lane));
          ok = (n * kTile + 8 * j + lane < len) && (PAGED ? p.km.valid(raw) : raw >= 0);
          const uint8_t* const rec = PAGED ? key_addr(p, raw) : p.kv + (int64_t)raw * kRecordBytes;
          *LDSP(uint64_t, tab + 8 * lane) = (uint64_t)(uintptr_t)(ok ? rec : zero);
        }
        const uint32_t bits = (uint32_t)__ballot(ok) & 0xFFu;
        if (lane == 0) *LDSP(uint8_t, keys + 4 * (n & (kRing - 1)) + j) = (uint8_t)bits;
      };
      // L: latent (4 token pairs; lanes 0..31 the even token, 32..63 the odd one,
      // whose lane position q loads chunk q ^ 8) and side data (scales + rope,
      // 9 chunks per token) of this wave's tokens into stage st.
      const uint32_t src_chunk = 16u * (uint32_t)((lane & 31) ^ ((lane >> 5) << 3));
      auto issue_tile = [&](int st) {
        uint64_t a[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) a[k] = *LDSP(uint64_t, tab + 8 * (2 * k + (lane >> 5)));
        const uint64_t s0 = *LDSP(uint64_t, tab + 8 * (lane / kSideChunks));
        const uint64_t s1 = *LDSP(uint64_t, tab + 8 * 7);
        const uint32_t dst = lat_at(st) + 4 * j * kPair;
#pragma unroll
        for (int k = 0; k < 4; ++k)
          dma16((const uint8_t*)(uintptr_t)(a[k] + src_chunk), __builtin_amdgcn_readfirstlane(dst + k * kPair));
        const uint32_t sd = side_at(st) + 8 * j * kSideTok;
        dma16((const uint8_t*)(uintptr_t)(s0 + kScaleOff + 16 * (lane % kSideChunks)), __builtin_amdgcn_readfirstlane(sd));
        // chunks 64 .. 71: token 7, pieces 1 .. 8
        if (lane < 8) dma16((const uint8_t*)(uintptr_t)(s1 + kScaleOff + 16 * (lane + 1)),
                            __builtin_amdgcn_readfirstlane(sd + 1024));
      };

      // ---- prologue: index tiles t0 .. t0+2, then records of tiles t0 .. t0+2,
      // each followed by the index tile three ahead.  From here on the issue
      // order is ... L(n) I(n+3) L(n+1) I(n+4) ..., so waiting for I(n+3) covers L(n).
      // index tiles t0 .. t0+2, unless the guessed ones are those
      if (!pref && !(spec && beg == beg_g && t0 == t0_g && t1 == t1_g)) {
        if (spec) wait_vm<0>();  // the guessed tiles land before the ring is refilled
#pragma unroll
        for (int k = 0; k < kAhead; ++k)
          if (t0 + k < t1) issue_idx(t0 + k);
      }
#pragma unroll
      for (int k = 0; k < kAhead; ++k) {
        if (t0 + k < t1) {
          // issued after I(t0+k): later index tiles, and L(t0+k') I(t0+k'+3) for k' < k
          int after = 0;
#pragma unroll
          for (int k2 = k + 1; k2 < kAhead; ++k2) after += t0 + k2 < t1;
#pragma unroll
          for (int k2 = 0; k2 < k; ++k2) after += kTileVm + (t0 + k2 + kAhead < t1);
          wait_vm_n(after);
          fill_table(t0 + k);
          issue_tile(k);
          if (t0 + k + kAhead < t1) issue_idx(t0 + k + kAhead);
        }
      }

      __syncthreads();  // the score waves' q exchange
      v4f O[4][8];  // O^T slices: dims 128j + 16dt + 4g + [0..3], head 16ht + t
      // heads 16ht + t: the streams' last references; O's reference is their max
      // (a stream's reference only rises, so that max is also O's running max)
      v4f rf0 = v4f{-INFINITY, -INFINITY, -INFINITY, -INFINITY}, rf1 = rf0;
      _Float16 fac[4];  // 2^(reference of this lane's stream - O's reference), exact
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        fac[ht] = (_Float16)0.0f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) O[ht][dt] = v4f{0, 0, 0, 0};
      }

      // transposed V reads: lane (t, g) loads token tv = 8g + t/2, bytes
      // 8(t&1) .. +7 of chunk 8j + dt (stored at (8j + dt) ^ 8 in odd rows)
      const int tv = 8 * g + (t >> 1);
      const uint32_t pv_off = row_off(tv) + 128 * (j ^ (tv & 1)) + 8 * (t & 1);

      int st_q = 0;  // stage of tile s (s - t0 mod kStages)
      for (int s = t0; s <= t1 + 1; ++s) {
        // this wave's records of tile s and index tile s+3 have landed: after
        // I(s+3) it queued L(x) I(x+3) for x = s+1, s+2 (those that exist)
        // (from step t1 on nothing of this unit is in flight)
        if (s + 2 * kAhead - 1 < t1) {
          wait_vm<(kAhead - 1) * (kTileVm + 1)>();  // every later tile exists
        } else if (s < t1) {
          int after = 0;
#pragma unroll
          for (int x = 1; x < kAhead; ++x) after += (s + x < t1 ? kTileVm : 0) + (s + x + kAhead < t1);
          wait_vm_n(after);
        }
        __syncthreads();
        const int st_l = st_q + kAhead >= kStages ? st_q + kAhead - kStages : st_q + kAhead;  // tile s+3
        __builtin_amdgcn_s_setprio(2);  // the gather ahead of the other role's work on this SIMD
        if (s + kAhead < t1) {
          fill_table(s + kAhead);
          issue_tile(st_l);
          if (s + 2 * kAhead < t1) issue_idx(s + 2 * kAhead);
        }
        __builtin_amdgcn_s_setprio(0);
        if (s > t0 + 1) {
          // ---- PV of tile s - 2: O^T[d, h] += V^T[d, tok] P'^T[tok, h]
          const int n = s - 2;
          const int b = n & 1;
          const int st_p = st_q >= 2 ? st_q - 2 : st_q + kStages - 2;
          const uint32_t vaddr = lat_at(st_p) + pv_off;
          v2i vr[8];
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) vr[dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDSP(v2i, vaddr + 16 * dt));
          const v8h sr = *LDSP(v8h, sx0 + b * kSxBuf + kPitch * j + 16 * g);
          // the streams' references of heads 16ht + t after tile n; when one
          // moved, O's reference (their max) and the streams' factors follow
          const v4f r0 = *LDSP(v4f, mx0 + b * kMxBuf + 16 * t);
          const v4f r1 = *LDSP(v4f, mx0 + b * kMxBuf + kHeads * 4 + 16 * t);
          // (references are integers or -inf: bit equality is equality)
          const v2u64 a0 = __builtin_bit_cast(v2u64, r0), a1 = __builtin_bit_cast(v2u64, r1);
          const v2u64 c0 = __builtin_bit_cast(v2u64, rf0), c1 = __builtin_bit_cast(v2u64, rf1);
          if (__builtin_amdgcn_ballot_w64(a0.x != c0.x || a0.y != c0.y || a1.x != c1.x || a1.y != c1.y)) {
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) {
              const float mo = fmax_(rf0[ht], rf1[ht]);
              const float mn = fmax_(r0[ht], r1[ht]);
              if (mo != -INFINITY && mn != mo) {
                const float al = __builtin_amdgcn_ldexpf(1.0f, (int)(mo - mn));
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) O[ht][dt] *= al;
              }
              // this lane's tokens 8g .. 8g+7 are stream g >> 1's
              const float rs = g < 2 ? r0[ht] : r1[ht];
              const float f = rs == -INFINITY ? 0.0f : __builtin_amdgcn_ldexpf(1.0f, (int)__builtin_fmaxf(rs - mn, -40.0f));
              fac[ht] = (_Float16)f;
            }
          }
          rf0 = r0;  // (unchanged unless a reference moved)
          rf1 = r1;
          v8h vh[8];
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) vh[dt] = cvt8_f16(vr[dt]);
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) {
            const v8h pr = *LDSP(v8h, px0 + b * kPxBuf + kPitch * (16 * ht + t) + 16 * g);
            const v8h pb = pr * (sr * fac[ht]);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) O[ht][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh[dt], pb, O[ht][dt], 0, 0, 0);
          }
        }
        st_q = st_q == kStages - 1 ? 0 : st_q + 1;
      }
      if (MULTI) {
        // the next unit's first index tiles (every ring slot is free by now),
        // landing during this unit's epilogue
        find_next();
        if (pref_next) {
#pragma unroll
          for (int k = 0; k < kAhead; ++k)
            if (un.t0 + k < un.t1) issue_idx_at(un.beg, un.t0 + k);
        }
      }
      __syncthreads();  // every head's {l, m} is written

      // ---- epilogue: this wave's 128 dims of every head (split: a partial
      // without the sink, which the combine folds in).  An unsplit row's bf16
      // output is staged in this wave's part of the (now idle) record stages, so
      // that consecutive lanes store consecutive bytes of a head's row.
      const uint32_t ob = lat_at(0) + j * (kHeads * kOutPitch);
      const KArgs ka = args();
      const float* const sink = SMLA_ARG(ka, sink);
      float* const lse_out = SMLA_ARG(ka, lse);
      float* const part_lse = SMLA_ARG(ka, part_lse);
      uint16_t* const part_o = SMLA_ARG(ka, part_o);
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const int hl = 16 * ht + t;  // head of the group
        const int h = h0 + hl;       // head of the row
        const bool h_ok = hl < Hl;
        // the two streams' sums, each relative to its own reference, at O's
        // reference (their max; every factor is an exact power of two)
        const v4f lmv = *LDSP(v4f, lm + 16 * hl);
        const float mo = fmax_(lmv.y, lmv.w);
        const float l = (lmv.y == -INFINITY ? 0.0f : lmv.x * __builtin_amdgcn_ldexpf(1.0f, (int)__builtin_fmaxf(lmv.y - mo, -200.0f))) +
                        (lmv.w == -INFINITY ? 0.0f : lmv.z * __builtin_amdgcn_ldexpf(1.0f, (int)__builtin_fmaxf(lmv.w - mo, -200.0f)));
        const Norm nm = finish_norm(l, mo, (split || !h_ok) ? -INFINITY : sink_log2(sink, h));
        if (j == 0 && g == 0 && h_ok) {
          if (split) part_lse[(int64_t)unit * H + h] = nm.lse2;
          else if (lse_out) lse_out[(int64_t)row * H + h] = nm.lse2 * kLn2;
        }
        if (split) {
          if (h_ok) {
            uint16_t* const po = part_o + ((int64_t)unit * H + h) * kLat + 128 * j;
            st_part16(po, g, &O[ht][0], nm.scale);
            st_part16(po + 64, g, &O[ht][4], nm.scale);
          }
        } else {
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            *LDSP(v2i, ob + kOutPitch * hl + 2 * (16 * dt + 4 * g)) = pack_bf16x4(O[ht][dt] * nm.scale);
        }
      }
      if (!split) {
        // this wave's rows back from LDS (the wave's own writes, which LDS
        // performs in order): 16 lanes per head, so each store instruction writes
        // four heads' 256 contiguous bytes
        asm volatile("" ::: "memory");
        uint16_t* const orow = SMLA_ARG(ka, out) + row * SMLA_ARG(ka, o_st) + 128 * j + 8 * (lane & 15);
        const int64_t o_sh = SMLA_ARG(ka, o_sh);
#pragma unroll
        for (int i = 0; i < kHeads / 4; ++i) {
          const int hl = 4 * i + (lane >> 4);
          const v4i v = *LDSP(v4i, ob + kOutPitch * hl + 16 * (lane & 15));
          if (hl < Hl) *(v4i*)(orow + (h0 + hl) * o_sh) = v;
        }
      }
      if (MULTI) wait_vm<0>();  // the stores, and the next unit's index tiles
      if (!MULTI || !has_next) return;
      // every wave is past this unit's epilogue (staged in the record
      // stages) before the next unit's q exchange and records land there
      __syncthreads();
      vb = vbn;
      u = un;
      pref = pref_next;
    }
  }
}
#undef SMLA_ARG

// With the plan and more units than the persistent grid (p.persist blocks,
// one per CU), the persistent kernel; otherwise one unit per block.
hipError_t launch_fwd_wide64(const FwdParams& p, Events ev, hipStream_t s) {
  const int64_t blocks = xcd_grid(p.T, p.S * p.hg);
  const bool multi = p.persist > 0 && p.desc != nullptr && blocks > p.persist;
  const dim3 grid((unsigned)(multi ? p.persist : blocks));
  auto go = [&](auto kernel) {
    hipExtLaunchKernelGGL(kernel, grid, dim3(w64::kThreads), 0, s, ev.start, ev.stop, 0, p);
  };
  if (p.km.paged) {
    if (multi) go(smla_fwdw64_kernel<true, true>);
    else go(smla_fwdw64_kernel<true, false>);
  } else {
    if (multi) go(smla_fwdw64_kernel<false, true>);
    else go(smla_fwdw64_kernel<false, false>);
  }
  return hipGetLastError();
}

}  // namespace smla
