// Wide-head forward for 17 <= H <= 32 heads (HT = 2 tiles of 16 heads; the
// kernel is written for HT tiles, and above 32 heads the forward uses the
// kernel of smla_wide64.hip).  Same method as the H <= 16 kernel
// (vLLM API page "vllm.models.kimi_k3.amd.ops.flydsl_sparse_mla_gfx950",
// module docstring; split chunks merged as on the K2-back page,
// stage_combine), laid out so that every record is converted once per head
// tile it meets and the MFMA units stay busy.
//
// One block of 8 waves (two per SIMD) per unit (row, chunk, head group); tiles of 64
// tokens, three LDS stages (records of tiles n+1 and n+2 are in flight while
// tile n is computed).
//   DMA: wave w brings in tokens 8w .. 8w+7 of a tile: their latent rows (token
//       pairs, odd rows swizzled as in the H <= 16 kernel) and their scales +
//       rope (144 B per token) into the tile's stage.
//   QK: wave w scores head tile w % HT against 16-token groups of the tile
//       (HT = 4: two groups per wave, HT = 2: one), q held in registers.
//   PV: wave w accumulates output dims 64w .. 64w+63 of every head over the
//       tile's 64 tokens (half a scale block: the V scale folds into P).
// P, the per-token V scales and the per-wave maxima go through LDS; two
// barriers per tile (records landed / scores written), a third only when
// the reference maximum moves.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_device.h"

namespace smla {
namespace nw {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;
constexpr int kStages = 3;
constexpr int kPair = 2 * kLat + 16;            // two latent rows + 16-B pad
constexpr int kLatStage = (kTile / 2) * kPair;  // 33,280 B
constexpr int kSideStage = kTile * kSideTok;    // 9,216 B
constexpr int kRingSlots = 8;                   // index ring (tiles)
constexpr int kPRow = 2 * kTile + 16;           // P / scale rows, f16, padded: 144 B
// Vector-memory instructions a wave issues per tile: 4 latent DMAs (token
// pairs) and 2 side DMAs (72 chunks of 16 B); an index DMA besides.
constexpr int kTileVm = 6;
constexpr int kQLoads = 18;                     // q loads per lane (16 latent + 2 rope)

template <int HT>
struct Cfg {
  static constexpr int kHeads = 16 * HT;
  static constexpr int kWph = kWaves / HT;         // waves per head tile
  static constexpr int kGpw = (kTile / 16) / kWph;  // 16-token QK groups per wave
  static constexpr int kLatOff = 0;
  static constexpr int kSideOff = kStages * kLatStage;
  static constexpr int kPxOff = kSideOff + kStages * kSideStage;  // P f16 [head][token]
  static constexpr int kSxOff = kPxOff + kHeads * kPRow;          // V scales f16 [block 4][token]
  static constexpr int kMxOff = kSxOff + 4 * kPRow;               // maxima f32 [head][wave of the tile]
  static constexpr int kRingOff = kMxOff + kHeads * kWph * 4;
  static constexpr int kTabOff = kRingOff + kRingSlots * kTile * 4;  // record addresses [wave][8]
  static constexpr int kKeyOff = kTabOff + kTile * 8;  // key masks u64 [ring slot]: bit i = token i is a key
  static constexpr int kBytes = kKeyOff + kRingSlots * 8;
  static_assert(kBytes <= 160 * 1024, "LDS budget");
  static_assert(kGpw >= 1 && kWph * kGpw * 16 == kTile, "QK covers the tile");
};

// vmcnt <= n for a wave-uniform n in [0, 8]
__device__ __forceinline__ void wait_vm_le8(int n) {
  switch (n) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    case 7: wait_vm<7>(); break;
    default: wait_vm<8>(); break;
  }
}

__device__ __forceinline__ uint32_t row_off(int tau) { return (tau >> 1) * kPair + (tau & 1) * kLat; }

}  // namespace nw

template <int HT>
__global__ __launch_bounds__(nw::kThreads, 1) void smla_fwdw_kernel(FwdParams p) {
  using namespace nw;
  using C = Cfg<HT>;
  __shared__ __attribute__((aligned(1024))) uint8_t s_lds[C::kBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 15;
  const int g = lane >> 4;
  const int ht = w % HT;        // QK head tile of this wave
  const int wi = w / HT;        // this wave's index among the waves of its head tile

  int rank, sub;
  if (p.hg == 1) fwd_unit(p.S, p.order == nullptr, rank, sub);  // one head group: sub is the chunk
  else xcd_unit(p.S * p.hg, rank, sub);
  if (rank >= p.T) return;
  const int chunk = sub % p.S;
  const int h0 = 64 * (sub / p.S);  // first head of this unit's head group

  const uint32_t base = lds_addr(s_lds);
  const int row = p.order ? p.order[rank] : rank;
  const int beg = p.indptr[row];
  const int len = max(p.indptr[row + 1] - beg, 0);
  const int tiles = unit_tiles<kThreads>(p, row, beg, len, kTile, (int*)(s_lds + C::kMxOff));
  const int ct = (tiles + p.S - 1) / p.S;
  const int t0 = min(chunk * ct, tiles);
  const int t1 = min(t0 + ct, tiles);
  const int unit = row * p.S + chunk;
  const bool split = p.S > 1;
  const int H = p.H;
  const int Hl = min(H - h0, C::kHeads);  // heads of this group

  if (t0 >= t1) {  // nothing to attend: zero output and the sink's lse, or an empty partial
    if (split) {
      for (int hh = h0 + tid; hh < h0 + Hl; hh += kThreads) p.part_lse[(int64_t)unit * H + hh] = -INFINITY;
    } else {
      for (int e = tid; e < Hl * (kLat / 8); e += kThreads) {
        const int hh = h0 + e / (kLat / 8), d = (e % (kLat / 8)) * 8;
        *(v4i*)(p.out + row * p.o_st + hh * p.o_sh + d) = v4i{0, 0, 0, 0};
      }
      if (p.lse)
        for (int hh = h0 + tid; hh < h0 + Hl; hh += kThreads)
          p.lse[(int64_t)row * H + hh] = p.sink ? p.sink[hh] : -INFINITY;
    }
    return;
  }

  const __amdgpu_buffer_rsrc_t irs = idx_rsrc(p.indices, p.idx_bytes);
  const uint8_t* const zero = p.zero;
  auto ring_at = [&](int n) -> uint32_t { return base + C::kRingOff + (n & (kRingSlots - 1)) * kTile * 4; };
  auto lat_at = [&](int st) -> uint32_t { return base + C::kLatOff + st * kLatStage; };
  auto side_at = [&](int st) -> uint32_t { return base + C::kSideOff + st * kSideStage; };
  const uint32_t tab = base + C::kTabOff + 64 * w;  // this wave's 8 record addresses

  // I: index DMA of this wave's 8 entries of tile n (bounded reads: positions
  // past nnz read 0; positions past the row are masked where they are used).
  auto issue_idx = [&](int n) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(ring_at(n) + 32 * w);
    if (lane < 8) buf_dma4(irs, (uint32_t)(beg + n * kTile + 8 * w + lane) * 4u, dst);
  };
  // record addresses of this wave's 8 tokens of tile n (no key: the zero
  // record), and their bits of the tile's key mask
  const uint32_t keys = base + C::kKeyOff;
  auto fill_table = [&](int n) {
    bool ok = false;
    if (lane < 8) {
      const int raw = *LDSP(int, ring_at(n) + 4 * (8 * w + lane));
      ok = (n * kTile + 8 * w + lane < len) && p.km.valid(raw);
      *LDSP(uint64_t, tab + 8 * lane) = (uint64_t)(uintptr_t)(ok ? key_addr(p, raw) : zero);
    }
    const uint32_t bits = (uint32_t)__ballot(ok) & 0xFFu;
    if (lane == 0) *LDSP(uint8_t, keys + 8 * (n & (kRingSlots - 1)) + w) = (uint8_t)bits;
  };
  // L: latent (4 token pairs; lanes 0..31 the even token, 32..63 the odd one,
  // whose lane position q loads chunk q ^ 8) and side data (scales + rope,
  // 9 chunks per token) of this wave's tokens of tile n into stage st.
  const uint32_t src_chunk = 16u * (uint32_t)((lane & 31) ^ ((lane >> 5) << 3));
  auto issue_tile = [&](int st) {
    uint64_t a[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *LDSP(uint64_t, tab + 8 * (2 * i + (lane >> 5)));
    const uint64_t s0 = *LDSP(uint64_t, tab + 8 * (lane / kSideChunks));
    const uint64_t s1 = *LDSP(uint64_t, tab + 8 * 7);
    const uint32_t dst = lat_at(st) + 4 * w * kPair;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16((const uint8_t*)(uintptr_t)(a[i] + src_chunk), __builtin_amdgcn_readfirstlane(dst + i * kPair));
    const uint32_t sd = side_at(st) + 8 * w * kSideTok;
    dma16((const uint8_t*)(uintptr_t)(s0 + kScaleOff + 16 * (lane % kSideChunks)), __builtin_amdgcn_readfirstlane(sd));
    // chunks 64 .. 71: token 7, pieces 1 .. 8
    if (lane < 8) dma16((const uint8_t*)(uintptr_t)(s1 + kScaleOff + 16 * (lane + 1)),
                        __builtin_amdgcn_readfirstlane(sd + 1024));
  };

  // ---- prologue: index tiles t0 .. t0+2 and this wave's q head tile (lane
  // (t, g): head 16 ht + t; latent K-step 2m / 2m+1 = dims 64m + 16g + [0..7] /
  // [8..15], rope K-step i = dims 512 + 32i + 8g + [0..7]); q of heads >= H is
  // loaded from head 0 (every lane issues the same loads) and zeroed after.
  issue_idx(t0);
  if (t0 + 1 < t1) issue_idx(t0 + 1);
  if (t0 + 2 < t1) issue_idx(t0 + 2);
  const int hq = 16 * ht + t;  // head of the group
  const bool hq_ok = hq < Hl;
  v4i qr[kQLoads];
  {
    const uint64_t qa = (uint64_t)(uintptr_t)(p.q + row * p.q_st + (int64_t)(h0 + (hq_ok ? hq : 0)) * p.q_sh);
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      gload16(qr[2 * m], qa + 2 * (64 * m + 16 * g));
      gload16(qr[2 * m + 1], qa + 2 * (64 * m + 16 * g + 8));
    }
    gload16(qr[16], qa + 2 * (kLat + 8 * g));
    gload16(qr[17], qa + 2 * (kLat + 32 + 8 * g));
  }
  wait_vm<0>();
#pragma unroll
  for (int i = 0; i < kQLoads; ++i) asm volatile("" : "+v"(qr[i]));
  v8bf qlat[16], qrope[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) qlat[i] = __builtin_bit_cast(v8bf, hq_ok ? qr[i] : v4i{0, 0, 0, 0});
#pragma unroll
  for (int i = 0; i < 2; ++i) qrope[i] = __builtin_bit_cast(v8bf, hq_ok ? qr[16 + i] : v4i{0, 0, 0, 0});
  // records of tiles t0 and t0+1, each followed by an index tile three ahead:
  // from here on the issue order is ... L(k) I(k+3) L(k+1) I(k+4) ...
  fill_table(t0);
  issue_tile(0);
  if (t0 + 3 < t1) issue_idx(t0 + 3);
  if (t0 + 1 < t1) {
    fill_table(t0 + 1);
    issue_tile(1);
    if (t0 + 4 < t1) issue_idx(t0 + 4);
  }

  float m_ref[HT], l_run[HT];  // per head 16j + t: reference max (log2 units), sum of P
  v4f O[HT][4];                // O^T slices: dims 64w + 16dt + 4g + [0..3], head 16j + t
#pragma unroll
  for (int j = 0; j < HT; ++j) {
    m_ref[j] = -INFINITY;
    l_run[j] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) O[j][dt] = v4f{0, 0, 0, 0};
  }

  const uint32_t px = base + C::kPxOff;
  const uint32_t sx = base + C::kSxOff;
  const uint32_t mx = base + C::kMxOff;
  // PV transposed reads (as in the H <= 16 kernel): lane (t, g) loads token
  // 32k + 8g + t/2, bytes 8(t&1) .. +7 of chunk 4w + dt (at (4w + dt) ^ 8 in odd rows)
  const int tv = 8 * g + (t >> 1);
  const uint32_t pv_off = row_off(tv) + 64 * (w ^ (2 * (tv & 1))) + 8 * (t & 1);
  const v2h ones = v2h{(_Float16)1.0f, (_Float16)1.0f};

  int st = 0;  // stage of tile n
  for (int n = t0; n < t1; ++n) {
    // this wave's records of tile n have landed; after them it queued at most
    // I(n+3), L(n+1) and I(n+4)
    wait_vm_le8((n + 3 < t1) + kTileVm * (n + 1 < t1) + (n + 4 < t1));
    // every wave's records of tile n have landed, and every wave is done with
    // tile n-1 (its stage, P, scales and maxima)
    __syncthreads();
    const int st2 = st == 0 ? 2 : st - 1;  // stage of tile n+2 (= tile n-1's)
    if (n + 2 < t1) {
      fill_table(n + 2);
      issue_tile(st2);
    }
    if (n + 5 < t1) issue_idx(n + 5);

    // ---- QK of this wave's groups: lane (t, g) gets head 16 ht + t, tokens 16j + 4g + r
    const uint32_t lat = lat_at(st);
    const uint32_t side = side_at(st);
    const uint64_t kmask = *LDSP(uint64_t, keys + 8 * (n & (kRingSlots - 1)));
    float x[C::kGpw][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int gi = 0; gi < C::kGpw; ++gi) {
      const int j = wi * C::kGpw + gi;  // 16-token group of the tile
      const int tok = 16 * j + t;       // the token whose K row this lane feeds
      const uint32_t qk_row = row_off(tok) + 16 * g;
      const uint32_t qk_a = qk_row + ((t & 1) ? 128u : 0u);
      const uint32_t qk_b = qk_row - ((t & 1) ? 128u : 0u);
      v4i kr[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) kr[m] = *LDSP(v4i, lat + ((m & 2) ? qk_b : qk_a) + 64 * m);
      const v4f ksc = *LDSP(v4f, side + kSideTok * tok);
      const v4i rp0 = *LDSP(v4i, side + kSideTok * tok + 16 + 16 * g);
      const v4i rp1 = *LDSP(v4i, side + kSideTok * tok + 16 + 64 + 16 * g);
      v4f acc0 = v4f{0, 0, 0, 0}, acc1 = v4f{0, 0, 0, 0};
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, rp0), qrope[0], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, rp1), qrope[1], acc1, 0, 0, 0);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float sc = ksc[m >> 1];
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
      const v4f S = acc0 + acc1;
      // which of tokens 16j + 4g + r are keys
      const uint32_t kb = (uint32_t)(kmask >> (16 * j + 4 * g));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[gi][r] = ((kb >> r) & 1u) ? S[r] * p.c_log2 : -INFINITY;
        tmax = fmax_(tmax, x[gi][r]);
      }
      // V scale of block g for token tok, clamped to 2^7, as f16 (one head tile writes it)
      if (ht == 0) *LDSP(_Float16, sx + kPRow * g + 2 * tok) = (_Float16)__builtin_fminf(ksc[g], kScaleCap);
    }
    tmax = xor_max(tmax);
    if (g == 0) *LDSP(float, mx + 4 * ((16 * ht + t) * C::kWph + wi)) = tmax;
    float m_own = m_ref[0];
#pragma unroll
    for (int j = 1; j < HT; ++j)
      if (j == ht) m_own = m_ref[j];
    // P of this wave's scores with the current reference (rewritten below if it moves)
    auto write_p = [&](float m_use) {
#pragma unroll
      for (int gi = 0; gi < C::kGpw; ++gi) {
        const int j = wi * C::kGpw + gi;
        _Float16 ph[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ph[r] = (_Float16)__builtin_amdgcn_exp2f(x[gi][r] - m_use + kShift);
        *LDSP(v2i, px + kPRow * (16 * ht + t) + 2 * (16 * j + 4 * g)) =
            __builtin_bit_cast(v2i, (v4h{ph[0], ph[1], ph[2], ph[3]}));
      }
    };
    write_p(m_own == -INFINITY ? 0.0f : m_own);
    __syncthreads();  // P, scales and maxima of tile n are written

    // ---- tile max of every head; the reference moves (for every head) when
    // some head's max exceeds it by more than kTau: the same decision in every wave
    {
      float M[HT];
      bool grow = false;
#pragma unroll
      for (int j = 0; j < HT; ++j) {
        M[j] = -INFINITY;
#pragma unroll
        for (int k = 0; k < C::kWph; ++k) M[j] = fmax_(M[j], *LDSP(float, mx + 4 * ((16 * j + t) * C::kWph + k)));
        grow |= M[j] > m_ref[j] + kTau;
      }
      if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
        for (int j = 0; j < HT; ++j) {
          const float m_new = fmax_(m_ref[j], M[j]);
          const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref[j] - m_new);
          if (__builtin_amdgcn_ballot_w64(m_ref[j] != -INFINITY)) {  // O and l are still zero otherwise
            l_run[j] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) O[j][dt] *= alpha;
          }
          m_ref[j] = m_new;
        }
        m_own = m_ref[0];
#pragma unroll
        for (int j = 1; j < HT; ++j)
          if (j == ht) m_own = m_ref[j];
        write_p(m_own == -INFINITY ? 0.0f : m_own);
        __syncthreads();
      }
    }

    // ---- PV: O^T[d, h] += V^T[d, tok] P'^T[tok, h] over the tile's 64 tokens;
    // l sums the same f16 P
    const uint32_t vaddr = lat + pv_off;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int tk = 32 * k + 8 * g;
      v2i vr[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        vr[dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDSP(v2i, vaddr + 16 * kPair * k + 16 * dt));
      const v8h sr = *LDSP(v8h, sx + kPRow * (w >> 1) + 2 * tk);
      v8h vh[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vh[dt] = cvt8_f16(vr[dt]);
#pragma unroll
      for (int j = 0; j < HT; ++j) {
        const v8h pr = *LDSP(v8h, px + kPRow * (16 * j + t) + 2 * tk);
        const v8h pb = pr * sr;
        l_run[j] = __builtin_amdgcn_fdot2(v2h{pr[0], pr[1]}, ones, l_run[j], false);
        l_run[j] = __builtin_amdgcn_fdot2(v2h{pr[2], pr[3]}, ones, l_run[j], false);
        l_run[j] = __builtin_amdgcn_fdot2(v2h{pr[4], pr[5]}, ones, l_run[j], false);
        l_run[j] = __builtin_amdgcn_fdot2(v2h{pr[6], pr[7]}, ones, l_run[j], false);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          O[j][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vh[dt], pb, O[j][dt], 0, 0, 0);
      }
    }
    st = st == 2 ? 0 : st + 1;
  }
  wait_vm_all();  // nothing is queued past the unit's last tile; this is a formality

  // ---- epilogue: every head's sum, then this wave's 64 dims of every head
  // (split: a partial without the sink, which the combine folds in)
#pragma unroll
  for (int j = 0; j < HT; ++j) {
    const int h = h0 + 16 * j + t;  // head of the row
    const bool h_ok = 16 * j + t < Hl;
    const float l = xor_sum(l_run[j]);
    const Norm nm = finish_norm(l, m_ref[j], (split || !h_ok) ? -INFINITY : sink_log2(p.sink, h));
    if (w == 0 && g == 0 && h_ok) {
      if (split) p.part_lse[(int64_t)unit * H + h] = nm.lse2;
      else if (p.lse) p.lse[(int64_t)row * H + h] = nm.lse2 * kLn2;
    }
    if (h_ok) {
      if (split) {
        st_part16(p.part_o + ((int64_t)unit * H + h) * kLat + 64 * w, g, O[j], nm.scale);
      } else {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int d = 64 * w + 16 * dt + 4 * g;
          *(v2i*)(p.out + row * p.o_st + h * p.o_sh + d) = pack_bf16x4(O[j][dt] * nm.scale);
        }
      }
    }
  }
}

template <int HT>
static hipError_t launch_fwdw_t(const FwdParams& p, Events ev, hipStream_t s) {
  const int64_t blocks = p.hg == 1 ? fwd_grid(p.T, p.S, p.order == nullptr) : xcd_grid(p.T, p.S * p.hg);
  hipExtLaunchKernelGGL((smla_fwdw_kernel<HT>), dim3((unsigned)blocks), dim3(nw::kThreads), 0, s,
                        ev.start, ev.stop, 0, p);
  return hipGetLastError();
}

hipError_t launch_fwd_wide(const FwdParams& p, Events ev, hipStream_t s) {
  const int ht = head_tiles(p.H);
  if (ht == 2) return launch_fwdw_t<2>(p, ev, s);
  if (ht >= 3 && ht <= 8) return launch_fwd_wide64(p, ev, s);  // above 64 heads: groups of 64
  return hipErrorInvalidValue;
}

}  // namespace smla
