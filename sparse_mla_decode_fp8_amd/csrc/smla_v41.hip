// DeepSeek V4.1 key records: forward (H <= 16) and the fused output
// epilogue.  Written from the K2-back page ("vllm.models.deepseek_v41.amd.
// mono.attention.back"):
//  * key_rec: a key's 576 data bytes (448 e4m3 nope values, then 64 bf16
//    rope values) at page + offset * 576, its 8 scale bytes at
//    page + page_records * 576 + offset * 8 (7 used: one E8M0 byte, i.e.
//    2^(byte - 127), per 64 nope dims);
//  * stage_split: K = [nope * scale, rope] over 512 dims and V the same 512
//    values, softmax in log2 units, chunk partials and their (max, sum);
//  * stage_combine: the chunks merged with the sink folded in, rounded to
//    bf16, the inverse GPT-J rotation of dims 448.. at the row's position,
//    and MXFP8 (E4M3 elements, one E8M0 scale per 32 values) of the result.
//    The pages do not define the MXFP8 rule; this is the OCP MX v1.0 one:
//    E = floor(log2 amax) - 8, elements clamped to +-448 and rounded to the
//    nearest E4M3 value (ties to even).
//
// The forward keeps the division of labour of the H <= 16 kernel
// (smla_kernels.hip): 8 waves, 128-token tiles, two LDS stages, QK split by
// 16-token groups and P.V by 64-dim output slices, P through LDS.  What
// differs:
//  * a token's LDS row is its 576 data bytes, the 16 rows a wave brings in
//    contiguous (9 DMA instructions of 64 x 16 B), with the 16-B chunk c of
//    token tau stored at c ^ ((tau >> 2) & 3) so that the QK reads and the
//    transposed P.V reads spread over all banks;
//  * the rope part of K is read from LDS, and the scale word (8 bytes from
//    the page's scale area) goes straight to registers;
//  * wave w < 7 owns nope dims 64w .. 64w+63, exactly one scale block, so the
//    V scale folds into P; wave 7 owns the rope dims (bf16 values, no scale);
//  * every unit writes a partial: the epilogue (merge, sink, bf16, rotation,
//    MXFP8) runs in the combine kernel, as on the page.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_device.h"

namespace smla {
namespace n41 {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 128;
constexpr int kNope = 448;
constexpr int kRow = 576;                       // data bytes of a key
constexpr int kLatStage = kTile * kRow;         // 73,728 B
constexpr int kIdxRing = 4;
constexpr int kPRow = 2 * kTile + 16;           // P / scale rows, f16, padded: 272 B
constexpr int kLatOff = 0;
constexpr int kPxOff = 2 * kLatStage;           // P f16 [head 16][token 128]
constexpr int kSxOff = kPxOff + 16 * kPRow;     // V scales f16 [block 8][token 128] (7 used)
constexpr int kMxOff = kSxOff + 8 * kPRow;      // tile maxima f32 [head 16][wave 8]
constexpr int kIdxRingOff = kMxOff + 16 * kWaves * 4;
constexpr int kTabOff = kIdxRingOff + kIdxRing * kTile * 4;  // {data, scale} u64 [2][token 128]
constexpr int kBytes = kTabOff + 2 * kTile * 16;
static_assert(kBytes <= 160 * 1024, "LDS budget");
// Vector-memory instructions a wave issues per tile: 9 data DMAs (16 rows of
// 36 chunks) and 1 scale-word load; an index DMA besides.
constexpr int kDataDma = 9;
constexpr int kTileVm = kDataDma + 1;
// q of the row is staged once per block in stage 1 (free until tile t0+1's
// records are queued): head hh's 512 bf16 at 1040 hh, the 16-byte pad putting
// the 16 heads a lane column reads in one instruction on distinct banks.
constexpr int kQPitch = 2 * 512 + 16;
static_assert(16 * kQPitch <= kLatStage, "q staging fits a stage");

__device__ __forceinline__ int swz(int tau) { return (tau >> 2) & 3; }
typedef short v4s16 __attribute__((ext_vector_type(4)));
typedef short v8s16 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void gload8(v2i& dst, uint64_t addr) {
  asm volatile("global_load_dwordx2 %0, %1, off" : "=v"(dst) : "v"(addr) : "memory");
}

// f32 2^(b - 127) of an E8M0 byte b (b = 0: 0.0, which the scaled conversion
// reads as the exponent field 0)
__device__ __forceinline__ float e8m0_f32(uint32_t b) { return __builtin_bit_cast(float, (b & 0xFFu) << 23); }

}  // namespace n41

// Data and scale-word addresses of a key entry (KeyMode::valid) in the paged
// V4.1 pools.
__device__ __forceinline__ void key_addr41(const FwdParams& p, int e, uint64_t& data, uint64_t& scale) {
  const bool c = e < 0;
  const uint32_t slot = (uint32_t)e & 0x7FFFFFFFu;
  const uint32_t sh = (uint32_t)(c ? p.pool_shift[1] : p.pool_shift[0]);
  const uint8_t* const base = c ? p.pool[1] : p.pool[0];
  const int64_t stride = c ? p.pool_stride[1] : p.pool_stride[0];
  const uint32_t off = slot & ((1u << sh) - 1u);
  const uint8_t* page = base + (int64_t)(slot >> sh) * stride;
  data = (uint64_t)(uintptr_t)(page + (int64_t)off * n41::kRow);
  scale = (uint64_t)(uintptr_t)(page + ((int64_t)1 << sh) * n41::kRow + (int64_t)off * 8);
}

// The fields the prologue needs first come as separate leading scalar
// arguments (preloaded into SGPRs at wave launch); `stride` > 0 is the slice
// stride nnz / T when there is no plan and nnz divides evenly, and lets each
// block queue its first index tiles before indptr arrives (queued again from
// the real start if the guess was wrong), as in the H <= 16 kernel.
__global__ __launch_bounds__(n41::kThreads, 1) void smla_fwd41_kernel(
    const int32_t* __restrict__ indptr, const int32_t* __restrict__ indices, const uint16_t* __restrict__ qbase,
    const int32_t* __restrict__ order, int32_t T, int32_t S, uint32_t idx_bytes, int32_t stride, FwdParams p) {
  using namespace n41;
  __shared__ __attribute__((aligned(1024))) uint8_t s_lds[kBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = lane & 15;
  const int g = lane >> 4;

  int rank, chunk;
  fwd_unit(S, order == nullptr, rank, chunk);
  if (rank >= T) return;

  const uint32_t base = lds_addr(s_lds);
  const __amdgpu_buffer_rsrc_t irs = idx_rsrc(indices, idx_bytes);
  auto ring_at = [&](int n) -> uint32_t { return base + kIdxRingOff + (n & (kIdxRing - 1)) * kTile * 4; };
  // I: this wave's 16 index entries of tile n of the slice starting at b
  // (bounded reads; positions past the row are masked in fill_table)
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

  const int row = order ? order[rank] : rank;
  const int beg = indptr[row];
  const int len = max(indptr[row + 1] - beg, 0);
  const int tiles = unit_tiles<kThreads>(p, row, beg, len, kTile, (int*)(s_lds + kMxOff));
  const int ct = (tiles + S - 1) / S;
  const int t0 = min(chunk * ct, tiles);
  const int t1 = min(t0 + ct, tiles);
  const int unit = row * S + chunk;
  const int H = p.H;
  const int h = t;
  const bool h_ok = h < H;

  if (t0 >= t1) {  // an empty partial: the combine gives the row out 0 and the sink's lse
    if (stride > 0) wait_vm_all();  // the speculative index DMA lands before the block ends
    for (int hh = tid; hh < H; hh += kThreads) p.part_lse[(int64_t)unit * H + hh] = -INFINITY;
    return;
  }

  const uint64_t zero = (uint64_t)(uintptr_t)p.zero;  // 656 zero bytes: data, then a zero scale word
  auto lat_at = [&](int st) -> uint32_t { return base + kLatOff + st * kLatStage; };
  auto tab_at = [&](int n) -> uint32_t { return base + kTabOff + (n & 1) * kTile * 16; };
  auto issue_idx = [&](int n) { issue_idx_at(beg, n); };
  // the data and scale addresses of this wave's 16 tokens of tile n (no key:
  // the zero record); returns the wave's valid-token mask
  auto fill_table = [&](int n) -> uint32_t {
    bool ok = false;
    if (lane < 16) {
      const int raw = *LDSP(int, ring_at(n) + 4 * (16 * w + lane));
      ok = (n * kTile + 16 * w + lane < len) && p.km.valid(raw);
      uint64_t d = zero, s = zero + kRow;
      if (ok) key_addr41(p, raw, d, s);
      *LDSP(v4i, tab_at(n) + 16 * (16 * w + lane)) =
          v4i{(int)(uint32_t)d, (int)(uint32_t)(d >> 32), (int)(uint32_t)s, (int)(uint32_t)(s >> 32)};
    }
    return (uint32_t)__ballot(ok) & 0xFFFFu;
  };
  // DMA lane map: instruction i, lane L carries chunk c = 64 i + L of this
  // wave's 16 contiguous rows: token c / 36, LDS chunk position c % 36, which
  // holds source chunk (c % 36) ^ swz(token).
  // per DMA i: the table byte offset of the lane's token (16 tk) in the high
  // half, the source byte offset in its record in the low half (the token
  // 16w + tk has the same swizzle as tk)
  uint32_t dma_map[kDataDma];
#pragma unroll
  for (int i = 0; i < kDataDma; ++i) {
    const uint32_t c = 64u * i + (uint32_t)lane;
    const uint32_t tk = c / 36u;
    dma_map[i] = ((16u * tk) << 16) | (16u * ((c - 36u * tk) ^ (uint32_t)swz((int)tk)));
  }
  auto issue_data = [&](int n, int st) {
    const uint32_t tab = tab_at(n) + 16 * (16 * w);
    const uint32_t dst = lat_at(st) + (16 * w) * kRow;
#pragma unroll
    for (int i = 0; i < kDataDma; ++i) {
      const uint64_t a = *LDSP(uint64_t, tab + (dma_map[i] >> 16));
      dma16((const uint8_t*)(uintptr_t)(a + (dma_map[i] & 0xFFFFu)), __builtin_amdgcn_readfirstlane(dst + 1024 * i));
    }
  };
  auto load_scales = [&](int n, v2i& sc) {
    const uint64_t a = *LDSP(uint64_t, tab_at(n) + 16 * (16 * w + t) + 8);
    gload8(sc, a);
  };

  // ---- prologue: index tiles t0 .. t0+2, and q of the row into stage 1
  // (wave w DMAs heads 2w and 2w+1, one 1 KB row each; heads >= H are not
  // loaded and their lanes use zeros)
  if (!(stride > 0 && beg == beg_g && t0 == t0_g)) {
    if (stride > 0) wait_vm_all();  // the guessed tiles land before the ring is refilled
    issue_idx(t0);
    if (t0 + 1 < t1) issue_idx(t0 + 1);
    if (t0 + 2 < t1) issue_idx(t0 + 2);
  }
  const uint32_t q_lds = lat_at(1);
  const int nq = (2 * w < H) + (2 * w + 1 < H);
  {
    const uint16_t* qrow = qbase + row * p.q_st;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int hh = 2 * w + j;
      if (hh < H)
        dma16((const uint8_t*)(qrow + (int64_t)hh * p.q_sh + 8 * lane),
              __builtin_amdgcn_readfirstlane(q_lds + kQPitch * hh));
    }
  }
  // this wave's index tiles have landed (its q rows, queued after them, may
  // not have: vector memory loads complete in issue order)
  if (nq == 2) wait_vm<2>();
  else if (nq == 1) wait_vm<1>();
  else wait_vm<0>();

  v2i scA, scB;   // scale words of this lane's QK token: tiles t0, t0+2, ... / t0+1, t0+3, ...
  uint32_t vmA = fill_table(t0), vmB = 0;
  if (t0 + 1 < t1) vmB = fill_table(t0 + 1);
  // tile t0's records alone, so that every block's first rows arrive as early
  // as they can; tile t0+1 follows when they have.  From here on the issue
  // order is ... L(n) I(n+3) L(n+1) I(n+4) ...
  issue_data(t0, 0);
  load_scales(t0, scA);
  wait_vm<kDataDma + 1>();  // this wave's q rows have landed (tile t0's rows may not)
  __syncthreads();          // every wave's have
  // q as bf16 B operands: head t, latent K-step 2m / 2m+1 = dims 64m + 16g +
  // [0..7] / [8..15] for m < 7, rope K-step i = dims 448 + 32i + 8g + [0..7]
  v8bf qk_b[16];
  {
    const uint32_t qr = q_lds + kQPitch * t;
#pragma unroll
    for (int m = 0; m < 7; ++m) {
      v4i a = *LDSP(v4i, qr + 2 * (64 * m + 16 * g));
      v4i b = *LDSP(v4i, qr + 2 * (64 * m + 16 * g + 8));
      if (!h_ok) a = b = v4i{0, 0, 0, 0};
      qk_b[2 * m] = __builtin_bit_cast(v8bf, a);
      qk_b[2 * m + 1] = __builtin_bit_cast(v8bf, b);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v4i a = *LDSP(v4i, qr + 2 * (kNope + 32 * i + 8 * g));
      if (!h_ok) a = v4i{0, 0, 0, 0};
      qk_b[14 + i] = __builtin_bit_cast(v8bf, a);
    }
  }
  if (t0 + 3 < t1) issue_idx(t0 + 3);
  // every wave has read q before tile t0+1's records are queued into stage 1
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __syncthreads();

  float m_ref = -INFINITY;
  float l_run = 0.0f;
  v4f O[4];       // O^T slices: dims 64w + 16dt + 4g + [0..3], head t
#pragma unroll
  for (int i = 0; i < 4; ++i) O[i] = v4f{0, 0, 0, 0};

  // QK reads: token 16w + t (swizzle (t >> 2) & 3), chunk 4m + g; rope chunks 28 + g, 32 + g
  const int sq = (t >> 2) & 3;
  const uint32_t qk_row = (16 * w + t) * kRow;
  // P.V transposed reads (waves 0..6): lane (t, g) loads token 32k + 8g + t/2,
  // bytes 8(t&1) .. +7 of chunk 4w + dt, found at (4w + dt) ^ swz(token) =
  // 4w + (dt ^ spv); lane (i, g) receives dim i of tokens 8g .. 8g+7.
  const int tv = 8 * g + (t >> 1);
  const int spv = (tv >> 2) & 3;
  const uint32_t pv_row = tv * kRow + 8 * (t & 1);
  uint32_t pv_off[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) pv_off[dt] = pv_row + 16 * (4 * w + (dt ^ spv));
  // rope P.V (wave 7): token 8g + 4h + t/4 of each 32-token step (swizzle
  // (2g + h) & 3), chunk 28 + (t&3)/2 (+ 2dt), byte 8(t&1) in it
  uint32_t rope_off[4][2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int tau = 8 * g + 4 * hh + (t >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
      rope_off[dt][hh] = tau * kRow + 16 * ((28 + 2 * dt + ((t & 3) >> 1)) ^ swz(tau)) + 8 * (t & 1);
  }
  const v2h ones = v2h{(_Float16)1.0f, (_Float16)1.0f};
  const uint32_t mx = base + kMxOff;
  const uint32_t px = base + kPxOff;
  const uint32_t sx = base + kSxOff;

  // One tile: n, its stage st (= (n - t0) & 1), its scale-word registers and key mask.
  auto tile = [&](int n, int st, v2i& sc, uint32_t& vmask) __attribute__((always_inline)) {
    const int left = t1 - n;
    // this wave's rows and scale word of tile n have landed (QK reads only the
    // rows this wave brought in); after them it queued at most I(n+3), L(n+1)
    // and I(n+4) -- for tile t0 only I(t0+3), then L(t0+1) and I(t0+4) here
    if (n == t0) {
      if (left >= 4) wait_vm<1>();
      else wait_vm<0>();
      if (left >= 2) {
        issue_data(n + 1, st ^ 1);
        load_scales(n + 1, scB);
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
    asm volatile("" : "+v"(sc));

    // ---- QK: lane (t, g) gets head t, tokens 16w + 4g + r
    const uint32_t lat = lat_at(st);
    v4f S;
    {
      v4i kr[7];
#pragma unroll
      for (int m = 0; m < 7; ++m) kr[m] = *LDSP(v4i, lat + qk_row + 16 * ((4 * m + g) ^ sq));
      const v4i rp0 = *LDSP(v4i, lat + qk_row + 16 * ((28 + g) ^ sq));
      const v4i rp1 = *LDSP(v4i, lat + qk_row + 16 * ((32 + g) ^ sq));
      // all nine reads are issued before the first conversion waits for one
      __builtin_amdgcn_sched_barrier(0);
      v4f acc0 = v4f{0, 0, 0, 0}, acc1 = v4f{0, 0, 0, 0};
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, rp0), qk_b[14], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, rp1), qk_b[15], acc1, 0, 0, 0);
#pragma unroll
      for (int m = 0; m < 7; ++m) {
        const float s = e8m0_f32((uint32_t)sc[m >> 2] >> (8 * (m & 3)));
        v2bf a0, a1, a2, a3, b0, b1, b2, b3;
        cvt4_bf16(kr[m].x, s, a0, a1);
        cvt4_bf16(kr[m].y, s, a2, a3);
        cvt4_bf16(kr[m].z, s, b0, b1);
        cvt4_bf16(kr[m].w, s, b2, b3);
        const v8bf ka = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
        const v8bf kb = {b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
        acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qk_b[2 * m], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qk_b[2 * m + 1], acc1, 0, 0, 0);
      }
      S = acc0 + acc1;
    }

    // ---- softmax (log2 domain) of this wave's 16 tokens
    float x[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = ((vmask >> (4 * g + r)) & 1u) ? S[r] * p.c_log2 : -INFINITY;
      tmax = fmax_(tmax, x[r]);
    }
    tmax = xor_max(tmax);
    if (g == 0) *LDSP(float, mx + 4 * (8 * t + w)) = tmax;
    auto write_p = [&](float m_use) {
      _Float16 ph[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ph[r] = (_Float16)__builtin_amdgcn_exp2f(x[r] - m_use + kShift);
      *LDSP(v2i, px + kPRow * t + 2 * (16 * w + 4 * g)) = __builtin_bit_cast(v2i, (v4h{ph[0], ph[1], ph[2], ph[3]}));
    };
    write_p(m_ref == -INFINITY ? 0.0f : m_ref);
    // V scales of blocks g and g + 4 (< 7) of token 16w + t, clamped to 2^7, as f16
    {
      const uint32_t b0 = (uint32_t)sc[0] >> (8 * g);
      *LDSP(_Float16, sx + kPRow * g + 2 * (16 * w + t)) = (_Float16)__builtin_fminf(e8m0_f32(b0), kScaleCap);
      if (g < 3) {
        const uint32_t b1 = (uint32_t)sc[1] >> (8 * g);
        *LDSP(_Float16, sx + kPRow * (g + 4) + 2 * (16 * w + t)) = (_Float16)__builtin_fminf(e8m0_f32(b1), kScaleCap);
      }
    }
    // tile n+2's table, while the other waves' rows may still be landing: its
    // index tile was queued before tile n's rows (which have landed), table
    // slot n & 1 was last read by tile n's own loads, and each wave touches
    // only its own entries of the ring and the table
    uint32_t vm_next = 0;
    if (left >= 3) vm_next = fill_table(n + 2);
    __syncthreads();

    // ---- tile max of head t over all waves; lazy reference move
    {
      const v2f mg = *LDSP(v2f, mx + 4 * (8 * t + 2 * g));
      const float M = xor_max(fmax_(mg.x, mg.y));
      if (__builtin_amdgcn_ballot_w64(M > m_ref + kTau)) {
        const float m_new = fmax_(m_ref, M);
        const float alpha = (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
        if (__builtin_amdgcn_ballot_w64(m_ref != -INFINITY)) {
          l_run *= alpha;
#pragma unroll
          for (int i = 0; i < 4; ++i) O[i] *= alpha;
        }
        m_ref = m_new;
        write_p(m_ref == -INFINITY ? 0.0f : m_ref);
        __syncthreads();
      }
    }

    // ---- PV over the tile's 128 tokens; l sums the same f16 P
    if (w < 7) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int tok = 32 * k + 8 * g;
        const v8h pr = *LDSP(v8h, px + kPRow * t + 2 * tok);
        const v8h sr = *LDSP(v8h, sx + kPRow * w + 2 * tok);
        const v8h pb = pr * sr;
        l_run = __builtin_amdgcn_fdot2(v2h{pr[0], pr[1]}, ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2(v2h{pr[2], pr[3]}, ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2(v2h{pr[4], pr[5]}, ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2(v2h{pr[6], pr[7]}, ones, l_run, false);
        v2i vr[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          vr[dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDSP(v2i, lat + 32 * kRow * k + pv_off[dt]));
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cvt8_f16(vr[dt]), pb, O[dt], 0, 0, 0);
      }
    } else {
      // rope dims (bf16, no scale fold): 16-bit transposed reads, lane (t, g)
      // loading token 32k + 8g + 4h + t/4, bytes 8(t&3) .. +7 of dims
      // 16dt .. 16dt+15 (chunk 28 + 2dt + (t&3)/2), so that lane (i, g)
      // receives dim 16dt + i of tokens 8g + 4h .. +3: the bf16 values are
      // the A operand as stored, against P rounded to bf16 (a relative error
      // of at most 2^-9 per weight; the softmax sum keeps the f16 P).
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int tok = 32 * k + 8 * g;
        const v8h pr = *LDSP(v8h, px + kPRow * t + 2 * tok);
        l_run = __builtin_amdgcn_fdot2(v2h{pr[0], pr[1]}, ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2(v2h{pr[2], pr[3]}, ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2(v2h{pr[4], pr[5]}, ones, l_run, false);
        l_run = __builtin_amdgcn_fdot2(v2h{pr[6], pr[7]}, ones, l_run, false);
        v8bf pbf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pbf[j] = (__bf16)(float)pr[j];
        v4s16 rv[4][2];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            rv[dt][hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDSP(v4s16, lat + 32 * kRow * k + rope_off[dt][hh]));
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const v8s16 a = __builtin_shufflevector(rv[dt][0], rv[dt][1], 0, 1, 2, 3, 4, 5, 6, 7);
          O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), pbf, O[dt], 0, 0, 0);
        }
      }
    }
    if (left == 1) return;  // the last tile: nothing reuses the stage or P

    __syncthreads();  // every wave is done with stage st, P, the scales and the maxima
    // ---- tile n+2 into stage st and these registers, then index tile n+5
    if (left >= 3) {
      vmask = vm_next;
      issue_data(n + 2, st);
      load_scales(n + 2, sc);
    }
    if (left >= 6) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // ring slot n+1 was read before its reload lands
      issue_idx(n + 5);
    }
  };

  for (int n = t0; n < t1; n += 2) {
    tile(n, 0, scA, vmA);
    if (n + 1 < t1) tile(n + 1, 1, scB, vmB);
  }
  wait_vm_all();

  // ---- epilogue: the unit's partial (normalised, without the sink) and its lse
  l_run = xor_sum(l_run);
  const Norm nm = finish_norm(l_run, m_ref, -INFINITY);
  if (w == 0 && g == 0 && h_ok) p.part_lse[(int64_t)unit * H + h] = nm.lse2;
  if (h_ok) st_part16(p.part_o + ((int64_t)unit * H + h) * kLat + 64 * w, g, O, nm.scale);
}

// ---------------------------------------------------------------- MXFP8

// A 32-value block is held by 4 lanes at lane stride 2 (8 values each):
// lanes q, q ^ 2, q ^ 4, q ^ 6 of each group of 8.
__device__ __forceinline__ float mx_block_amax(float a) {
  a = fmax_(a, __shfl_xor(a, 2));
  return fmax_(a, __shfl_xor(a, 4));
}
// E8M0 byte E + 127 with E = floor(log2 amax) - 8 (at least -127), and the
// exact multiplier 2^-E.
__device__ __forceinline__ uint32_t mx_code(float amax) {
  const int e = (int)((__builtin_bit_cast(uint32_t, amax) >> 23) & 0xFF);  // biased exponent
  const int code = e - 8;  // (e - 127 - 8) + 127; a zero or subnormal amax gives e = 0
  return (uint32_t)(code < 0 ? 0 : code);
}
__device__ __forceinline__ float mx_mul(uint32_t code) {  // 2^(127 - code), code in [0, 254]
  return __builtin_bit_cast(float, (254u - code) << 23);
}
// Eight values times mul, clamped to +-448, as E4M3 codes (round to nearest even).
__device__ __forceinline__ v2i mx_pack8(const float y[8], float mul) {
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = __builtin_fminf(__builtin_fmaxf(y[i] * mul, -448.0f), 448.0f);
  int w0 = 0, w1 = 0;
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], w0, false);
  w0 = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], w0, true);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], w1, false);
  w1 = __builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], w1, true);
  return v2i{w0, w1};
}

// ---------------------------------------------------------------- combine + epilogue

// One wave per (row, head); lane L holds partial positions 8L .. 8L+7, i.e.
// dims part_dim(8L) + [0..3] and part_dim(8L + 4) + [0..3].  Lanes with the
// same 32-dim MXFP8 block sit at lane stride 2 (positions 16g + 4dt: dt in
// {0, 1} or {2, 3} of one 64-dim block).
// The merge of one (row, head): chunk statistics and partials are all loaded
// before any is used (slots past S re-read chunk 0 and are ignored).
// The rope lanes' cos / sin (4 pairs) are loaded right behind the partials,
// so that their dependent loads (position, then table) overlap the partials'.
template <int SMAX>
__device__ __forceinline__ void merge41(const float* __restrict__ part_lse, const uint16_t* __restrict__ part_o,
                                        int H, int S, int64_t u0, int h, int lane, float sink2,
                                        const Combine41Params& p, int row, bool rope, int d0, int d1,
                                        float acc[8], float& M, float& L, float cr[4], float sr[4]) {
  float lc[SMAX];
  v4i raw[SMAX];
#pragma unroll
  for (int c = 0; c < SMAX; ++c) {
    const int64_t u = u0 + (c < S ? c : 0);
    lc[c] = part_lse[u * H + h];
    raw[c] = *(const v4i*)(part_o + (u * H + h) * kLat + 8 * lane);
  }
  {
    const int pos = min(max(p.pos[row], 0), p.n_pos - 1);
    const float* cs = p.cos_sin + (int64_t)pos * 64;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int pr0 = rope ? ((half ? d1 : d0) - n41::kNope) >> 1 : 0;  // first pair index of the piece
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        cr[2 * half + j] = cs[pr0 + j];
        sr[2 * half + j] = cs[32 + pr0 + j];
      }
    }
  }
  M = sink2;
#pragma unroll
  for (int c = 0; c < SMAX; ++c)
    if (c < S) M = fmax_(M, lc[c]);
  L = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  if (M == -INFINITY) return;
  L = __builtin_amdgcn_exp2f(sink2 - M);
#pragma unroll
  for (int c = 0; c < SMAX; ++c) {
    if (c < S && lc[c] != -INFINITY) {  // an empty chunk's partial was never written
      const float wgt = __builtin_amdgcn_exp2f(lc[c] - M);
      L += wgt;
      const v4f lo = half4_to_f32(v2i{raw[c].x, raw[c].y});
      const v4f hi = half4_to_f32(v2i{raw[c].z, raw[c].w});
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += wgt * lo[i];
        acc[4 + i] += wgt * hi[i];
      }
    }
  }
}

// The partials, the row order and the sizes come as separate leading
// arguments, preloaded into SGPRs at wave launch.
__global__ __launch_bounds__(256) void smla_combine41_kernel(
    const float* __restrict__ part_lse, const uint16_t* __restrict__ part_o, const int32_t* __restrict__ order,
    int32_t T, int32_t H, int32_t S, Combine41Params p) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  int rank, hq;
  xcd_unit((H + 3) / 4, rank, hq);
  const int h = 4 * hq + wv;
  if (rank >= T || h >= H) return;
  const int row = order ? order[rank] : rank;
  const int64_t u0 = (int64_t)row * S;
  // merge (K2-back page, stage_combine): M = max(max_c lse2_c, sink2)
  const float sink2 = p.sink ? p.sink[h] * 1.4426950408889634f : -INFINITY;
  const int d0 = part_dim(8 * lane), d1 = part_dim(8 * lane + 4);
  const bool rope = d0 >= n41::kNope;  // both pieces of this lane are rope dims (one 64-dim block)
  float acc[8], M, L, cr[4], sr[4];
  if (S <= 4) merge41<4>(part_lse, part_o, H, S, u0, h, lane, sink2, p, row, rope, d0, d1, acc, M, L, cr, sr);
  else if (S <= 8) merge41<8>(part_lse, part_o, H, S, u0, h, lane, sink2, p, row, rope, d0, d1, acc, M, L, cr, sr);
  else if (S <= 16) merge41<16>(part_lse, part_o, H, S, u0, h, lane, sink2, p, row, rope, d0, d1, acc, M, L, cr, sr);
  else merge41<32>(part_lse, part_o, H, S, u0, h, lane, sink2, p, row, rope, d0, d1, acc, M, L, cr, sr);
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  // bf16, then the inverse GPT-J rotation of the rope dims (448 ..)
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = round_bf16(acc[i] * inv);
  if (rope) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float c = cr[2 * half + j], s = sr[2 * half + j];
        const float e = y[4 * half + 2 * j], o = y[4 * half + 2 * j + 1];
        y[4 * half + 2 * j] = e * c + o * s;
        y[4 * half + 2 * j + 1] = o * c - e * s;
      }
    }
  }
  if (p.y_out) {
    float* yo = p.y_out + ((int64_t)row * p.H + h) * kLat;
    *(v4f*)(yo + d0) = v4f{y[0], y[1], y[2], y[3]};
    *(v4f*)(yo + d1) = v4f{y[4], y[5], y[6], y[7]};
  }
  // MXFP8 of each 32 dims
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmax_(am, __builtin_fabsf(y[i]));
  am = mx_block_amax(am);
  const uint32_t code = mx_code(am);
  const v2i q8 = mx_pack8(y, mx_mul(code));
  uint8_t* xo = p.xo + ((int64_t)row * p.H + h) * kLat;
  *(int*)(xo + d0) = q8.x;
  *(int*)(xo + d1) = q8.y;
  // block index of this lane's dims: (d0 / 32); one lane of the four writes it
  if (((lane >> 1) & 3) == 0) p.xos[((int64_t)row * p.H + h) * (kLat / 32) + d0 / 32] = (uint8_t)code;
  if (lane == 0 && p.lse) p.lse[(int64_t)row * p.H + h] = L > 0.0f ? (M + __builtin_log2f(L)) * kLn2 : -INFINITY;
}

// Test hook: MXFP8 of n f32 values (n a multiple of 64) with the combine's
// own lane layout and helpers: wave b takes values 64b .. 64b+63 as two
// 32-value blocks, lane L values 64b + part_pos(L) .. +7 where the block of
// lane L is (L & 1) and its 8 values are the ((L >> 1) & 3)-th eighth; lanes
// 8 .. 63 repeat lanes 0 .. 7's blocks at the next values.
__global__ __launch_bounds__(64) void smla_mxfp8_kernel(const float* y, int64_t n, uint8_t* codes, uint8_t* scales) {
  const int lane = threadIdx.x;
  const int64_t b = blockIdx.x;  // 512 values per wave: 8 groups of 8 lanes x 64 values
  const int grp = lane >> 3;     // 64-value group of this lane
  const int q = lane & 7;
  const int blk = q & 1, part = q >> 1;  // block of the group, eighth of the block
  const int64_t v0 = b * 512 + grp * 64 + blk * 32 + part * 8;
  if (b * 512 + grp * 64 >= n) return;  // whole groups only (n is a multiple of 64)
  float yy[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) yy[i] = y[v0 + i];
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) am = fmax_(am, __builtin_fabsf(yy[i]));
  am = mx_block_amax(am);
  const uint32_t code = mx_code(am);
  const v2i q8 = mx_pack8(yy, mx_mul(code));
  *(v2i*)(codes + v0) = q8;
  if (part == 0) scales[v0 / 32] = (uint8_t)code;
}

// ---------------------------------------------------------------- launchers

hipError_t launch_fwd41(const FwdParams& p, Events ev, hipStream_t s) {
  const int64_t blocks = fwd_grid(p.T, p.S, p.order == nullptr);
  hipExtLaunchKernelGGL(smla_fwd41_kernel, dim3((unsigned)blocks), dim3(n41::kThreads), 0, s, ev.start, ev.stop, 0,
                        p.indptr, p.indices, p.q, p.order, p.T, p.S, p.idx_bytes, p.stride, p);
  return hipGetLastError();
}

hipError_t launch_combine41(const Combine41Params& p, Events ev, hipStream_t s) {
  const int64_t blocks = xcd_grid(p.T, (p.H + 3) / 4);
  hipExtLaunchKernelGGL(smla_combine41_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ev.start, ev.stop, 0,
                        p.part_lse, p.part_o, p.order, p.T, p.H, p.S, p);
  return hipGetLastError();
}

hipError_t launch_mxfp8(const float* y, int64_t n, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t blocks = (n + 511) / 512;
  hipLaunchKernelGGL(smla_mxfp8_kernel, dim3((unsigned)blocks), dim3(64), 0, s, y, n, codes, scales);
  return hipGetLastError();
}

}  // namespace smla
