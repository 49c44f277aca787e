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
// Design for MI355X (differs from the FlyDSL kernel; reasons in the design doc):
//  * plan kernel: per-row tile counts (a bounded scan for the last valid entry
//    when has_invalid) and a longest-first row order (counting sort).
//  * forward kernel: a workgroup owns one (row, chunk) unit.  Waves are
//    (head tile of 16, token group of 32 tokens).  Every wave runs QK, online
//    softmax and PV over all 512 dims for its own 32 tokens, so tiles need no
//    cross-wave exchange; token groups merge once per unit through LDS.
//  * the latent tile arrives by LDS DMA (global_load_lds_dwordx4 from 64-bit
//    per-lane record addresses), double-buffered per wave; scales and rope go
//    straight to registers.  Masked positions read a zero record.
//  * QK: K dequantised exactly to bf16 by v_cvt_scalef32_pk_bf16_fp8 with the
//    record's pow2 scale (the conversion applies the scale's exponent only),
//    bf16 MFMA 16x16x32 against bf16 q (rope the same).
//  * PV: V read transposed from LDS (ds_read_b64_tr_b8), converted exactly
//    e4m3 -> f16, f16 MFMA 16x16x32; the per-token V scale is folded into P.
//    The QK output layout (lane = head, 4 token rows) is chosen so each lane's
//    scores are already its PV B operand: P never moves between lanes.
//  * combine kernel: LSE merge of the chunks of split rows.
//  * workgroup -> unit mapping is XCD-aware: all chunks of a row run on one XCD
//    (dispatch is round-robin over the 8 XCDs), so partials and q stay in that
//    XCD's L2.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "smla_internal.h"

namespace smla {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

#define LDSP(T, off) ((__attribute__((address_space(3))) T*)(uintptr_t)(off))

constexpr int kLat = 512;
constexpr int kScaleOff = 512;
constexpr int kRopeOff = 528;
constexpr int kWaveLatBytes = kTokensPerWave * kLat;  // 16 KiB per wave per stage
constexpr float kPShift = 8.0f;
constexpr float kScaleCap = 128.0f;  // 2^7: P' = P * scale <= 2^15 fits f16
constexpr float kLn2 = 0.693147180559945309f;
constexpr int kMergeRow = kLat + 4;  // padded f32 row of the LDS merge area

// A record of zeros: masked positions gather it, so they read finite data
// (V = 0, scale = 0) wherever the cache is, and never address row 0.
__device__ __attribute__((aligned(256))) uint8_t g_zero_record[kRecordBytes];

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t idx_rsrc(const int32_t* base, uint32_t nbytes) {
  // raw buffer, stride 0: reads at byte offsets >= nbytes return 0
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)nbytes, 0x00020000);
}

__device__ __forceinline__ int load_idx(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, 0);
}

// 16 bytes from a 64-bit global address into LDS at lds_base + 16*lane (LDS
// DMA).  Issued from asm so the compiler's wait-count insertion does not make
// every later LDS read wait for it; callers wait explicitly (vmcnt(0)).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is the DMA's LDS base; nothing else here uses it
__device__ __forceinline__ void dma16(const uint8_t* src, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

// vmcnt(0) only (expcnt, lgkmcnt left at their maxima), through the intrinsic
// so the compiler's own wait tracking knows every load has completed here.
__device__ __forceinline__ void wait_vm_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ float fmax_(float a, float b) { return __builtin_fmaxf(a, b); }

__device__ __forceinline__ float xor_max(float v) {
  v = fmax_(v, __shfl_xor(v, 16));
  return fmax_(v, __shfl_xor(v, 32));
}
__device__ __forceinline__ float xor_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (uint16_t)((u >> 16) | ((u & 0xffff) ? 0x40 : 0));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 4 e4m3 codes (one word) x pow2 scale -> 4 bf16 (exact), as two v2bf.
__device__ __forceinline__ void cvt4_bf16(int w, float sc, v2bf& lo, v2bf& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, sc, true);
}

// 8 e4m3 codes (two words) -> 8 f16 (exact).
__device__ __forceinline__ v8h cvt8_f16(v2i w) {
  v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, false);
  v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.x, 1.0f, true);
  v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, false);
  v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.y, 1.0f, true);
  return v8h{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ const uint8_t* record_ptr(const uint8_t* kv, int ix) {
  return ix >= 0 ? kv + (int64_t)ix * kRecordBytes : g_zero_record;
}

// XCD-aware unit mapping: block b runs on XCD b % 8; rows of rank r go to XCD
// r % 8 and the `per_row` blocks of a row are consecutive on that XCD.
__device__ __forceinline__ void xcd_unit(int per_row, int& rank, int& sub) {
  const int b = blockIdx.x;
  const int i = b >> 3;
  rank = (b & 7) + 8 * (i / per_row);
  sub = i % per_row;
}

// ---------------------------------------------------------------- plan

// One wave per row: tile count (after the has_invalid trim); the last block to
// finish sorts rows by tile count, longest first (FlyDSL page: long rows are
// issued first so the long tail starts early).
__global__ __launch_bounds__(256) void smla_plan_kernel(PlanParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  __shared__ int s_last;
  __shared__ int s_hist[kPlanBuckets];
  if (row < p.T) {
    const int beg = p.indptr[row];
    const int len = max(p.indptr[row + 1] - beg, 0);
    int eff = len;
    if (p.has_invalid) {
      const __amdgpu_buffer_rsrc_t r = idx_rsrc(p.indices, p.idx_bytes);
      int lastp = 0;
      for (int base = 0; base < len; base += 256) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int pos = base + 4 * lane + j;
          const int v = load_idx(r, (uint32_t)(beg + pos) * 4u);
          if (pos < len && v >= 0) lastp = pos + 1;
        }
      }
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) lastp = max(lastp, __shfl_xor(lastp, sh));
      eff = lastp;
    }
    if (lane == 0) p.row_tiles[row] = (eff + p.tile - 1) / p.tile;
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int i = threadIdx.x; i < kPlanBuckets; i += blockDim.x) s_hist[i] = 0;
  __syncthreads();
  for (int r = threadIdx.x; r < p.T; r += blockDim.x) {
    const int t = __hip_atomic_load(p.row_tiles + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    atomicAdd(&s_hist[min(t, kPlanBuckets - 1)], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // exclusive prefix, largest bucket first
    int acc = 0;
    for (int b = kPlanBuckets - 1; b >= 0; --b) {
      const int c = s_hist[b];
      s_hist[b] = acc;
      acc += c;
    }
  }
  __syncthreads();
  for (int r = threadIdx.x; r < p.T; r += blockDim.x) {
    const int t = __hip_atomic_load(p.row_tiles + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    p.order[atomicAdd(&s_hist[min(t, kPlanBuckets - 1)], 1)] = r;
  }
  if (threadIdx.x == 0) __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- forward

template <int HT, int TG>
struct FwdCfg {
  static constexpr int kWaves = HT * TG;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kTile = kTokensPerWave * TG;
  static constexpr int kLatBytes = 2 * TG * kWaveLatBytes;  // 2 stages
  static constexpr int kMergeBytes = TG > 1 ? TG * HT * 16 * kMergeRow * 4 : 0;
  static constexpr int kBigBytes = kLatBytes > kMergeBytes ? kLatBytes : kMergeBytes;
};

struct Side {
  v4f sc[2];     // 4 block scales of tokens t and 16 + t
  v4i rp[2][2];  // rope A operands: [subtile][rope K-step]
};

template <int HT, int TG>
__global__ __launch_bounds__(64 * HT * TG, 1) void smla_fwd_kernel(FwdParams p) {
  using C = FwdCfg<HT, TG>;
  __shared__ __attribute__((aligned(1024))) uint8_t s_big[C::kBigBytes];
  __shared__ __attribute__((aligned(16))) v4f s_ks[C::kWaves][kTokensPerWave];
  __shared__ float s_m[C::kWaves][16];
  __shared__ float s_l[C::kWaves][16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ht = wave % HT;
  const int tg = wave / HT;
  const int t = lane & 15;  // QK token row / PV dim row / C column = head
  const int g = lane >> 4;  // lane group

  int rank, chunk;
  xcd_unit(p.S, rank, chunk);
  if (rank >= p.T) return;
  const int row = p.order[rank];
  const int beg = p.indptr[row];
  const int len = max(p.indptr[row + 1] - beg, 0);
  const int tiles = p.row_tiles[row];
  const int ct = (tiles + p.S - 1) / p.S;
  const int t0 = min(chunk * ct, tiles);
  const int t1 = min(t0 + ct, tiles);
  const int unit = row * p.S + chunk;
  const bool split = p.S > 1;

  const int h = 16 * ht + t;
  const bool h_ok = h < p.H;

  if (t0 >= t1) {  // nothing to attend: zero output / -inf lse, or an empty partial
    if (split) {
      for (int hh = tid; hh < p.H; hh += C::kThreads) p.part_lse[(int64_t)unit * p.H + hh] = -INFINITY;
    } else {
      for (int e = tid; e < p.H * (kLat / 8); e += C::kThreads) {
        const int hh = e / (kLat / 8), d = (e % (kLat / 8)) * 8;
        *(v4i*)(p.out + row * p.o_st + hh * p.o_sh + d) = v4i{0, 0, 0, 0};
      }
      if (p.lse)
        for (int hh = tid; hh < p.H; hh += C::kThreads) p.lse[(int64_t)row * p.H + hh] = -INFINITY;
    }
    return;
  }

  // ---- q as bf16 B operands.  Latent K-step 2m / 2m+1: dims 64m + 16g + [0..7] / [8..15];
  // rope K-step i: dims 512 + 32i + 8g + [0..7].
  v8bf qlat[16];
  v8bf qrope[2];
  {
    const uint16_t* qr = p.q + row * p.q_st + (int64_t)(h_ok ? h : 0) * p.q_sh;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      v4i a = *(const v4i*)(qr + 64 * m + 16 * g);
      v4i b = *(const v4i*)(qr + 64 * m + 16 * g + 8);
      if (!h_ok) a = b = v4i{0, 0, 0, 0};
      qlat[2 * m] = __builtin_bit_cast(v8bf, a);
      qlat[2 * m + 1] = __builtin_bit_cast(v8bf, b);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v4i a = *(const v4i*)(qr + kLat + 32 * i + 8 * g);
      if (!h_ok) a = v4i{0, 0, 0, 0};
      qrope[i] = __builtin_bit_cast(v8bf, a);
    }
  }

  const __amdgpu_buffer_rsrc_t irs = idx_rsrc(p.indices, p.idx_bytes);
  const uint32_t lat0 = lds_addr(s_big) + tg * kWaveLatBytes;  // stage st adds st*TG*16K

  // Index of token (lane & 31) of this wave's 32 positions in tile n.  The raw
  // (bounded) load and the row-end mask are separate so a prefetched index is
  // not consumed, and so not waited for, before the next tile.
  auto pos_of = [&](int n) -> int { return n * C::kTile + kTokensPerWave * tg + (lane & 31); };
  auto load_raw = [&](int n) -> int { return load_idx(irs, (uint32_t)(beg + pos_of(n)) * 4u); };
  auto masked = [&](int raw, int n) -> int { return pos_of(n) < len ? raw : -1; };
  // Latent DMA of the wave's 32 tokens into stage `st`.  LDS holds token tau's
  // 16-byte chunk c at slot c ^ tau of its 512-byte row; instruction k covers
  // tokens 2k, 2k+1 (lane -> token 2k + lane/32, slot lane % 32).
  auto issue_dma = [&](int ix_lane, int st) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lat0 + st * TG * kWaveLatBytes);
#pragma unroll
    for (int k = ht; k < 16; k += HT) {
      const int v0 = __builtin_amdgcn_readlane(ix_lane, 2 * k);
      const int v1 = __builtin_amdgcn_readlane(ix_lane, 2 * k + 1);
      const int tau = 2 * k + (lane >> 5);
      const uint8_t* rec = record_ptr(p.kv, (lane >> 5) ? v1 : v0);
      dma16(rec + 16 * ((lane & 31) ^ tau), base + 1024 * k);
    }
  };
  auto load_side = [&](int ix_lane, Side& sd) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint8_t* rec = record_ptr(p.kv, __shfl(ix_lane, 16 * s + t));
      sd.sc[s] = *(const v4f*)(rec + kScaleOff);
      sd.rp[s][0] = *(const v4i*)(rec + kRopeOff + 16 * g);
      sd.rp[s][1] = *(const v4i*)(rec + kRopeOff + 64 + 16 * g);
    }
  };

  float m_run = -INFINITY;
  float l_run = 0.0f;
  v4f O[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) O[i] = v4f{0, 0, 0, 0};

  int raw_cur = load_raw(t0);
  {
    const int ix0 = masked(raw_cur, t0);
    issue_dma(ix0, 0);
  }
  Side sd_next;
  load_side(masked(raw_cur, t0), sd_next);
  int raw_next = load_raw(t0 + 1);

  // PV transposed-read lane address: lane (t, g) reads token row j = t/2,
  // tau_j = 16(j/4) + 4g + j%4, byte half t%2; the dim chunk dt is XORed in.
  const int jrow = t >> 1;
  const int tau_v = 16 * (jrow >> 2) + 4 * g + (jrow & 3);
  const uint32_t v_off = 512 * tau_v + 16 * tau_v + 8 * (t & 1);

  for (int n = t0; n < t1; ++n) {
    const int st = (n - t0) & 1;
    wait_vm_all();            // tile n's DMA and side data have landed
    if (HT > 1) __syncthreads();  // ... for every wave sharing the tile
    const int ix_n = masked(raw_cur, n);
    const Side sd = sd_next;
    if (n + 1 < t1) {         // prefetch tile n+1 into the other stage
      const int ix1 = masked(raw_next, n + 1);
      issue_dma(ix1, st ^ 1);
      load_side(ix1, sd_next);
      raw_cur = raw_next;
      raw_next = load_raw(n + 2);  // bounded read; masked when used
    }
    const uint32_t lat = lat0 + st * TG * kWaveLatBytes;
    const uint32_t vmask = (uint32_t)__ballot(ix_n >= 0);  // bit tau: token tau is a key

    // ---- QK: S^T tiles; lane (t, g) gets head t, tokens 16s + 4g + r.
    v4f S[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int tau = 16 * s + t;
      const uint32_t kb = lat + 512 * tau + 16 * tau;
      v4f acc = v4f{0, 0, 0, 0};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const v4i raw = *LDSP(v4i, kb ^ (16 * (4 * m + g)));
        const float sc = sd.sc[s][m >> 1];
        v2bf a0, a1, a2, a3, b0, b1, b2, b3;
        cvt4_bf16(raw.x, sc, a0, a1);
        cvt4_bf16(raw.y, sc, a2, a3);
        cvt4_bf16(raw.z, sc, b0, b1);
        cvt4_bf16(raw.w, sc, b2, b3);
        const v8bf ka = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
        const v8bf kb8 = {b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qlat[2 * m], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb8, qlat[2 * m + 1], acc, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, sd.rp[s][i]), qrope[i], acc, 0, 0, 0);
      S[s] = acc;
    }

    // ---- online softmax (log2 domain), per head over this wave's tokens
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tau = 16 * s + 4 * g + r;
        const float v = ((vmask >> tau) & 1u) ? S[s][r] * p.c_log2 : -INFINITY;
        x[4 * s + r] = v;
        tmax = fmax_(tmax, v);
      }
    tmax = xor_max(tmax);
    const float m_new = fmax_(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float P[8];
    float psum = 0.0f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      P[k] = __builtin_amdgcn_exp2f(x[k] - m_use + kPShift);
      psum += P[k];
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < 32; ++i) O[i] *= alpha;

    // ---- V scales of this lane's 8 tokens (wave-local exchange through LDS)
    if (g == 0) {
      s_ks[wave][t] = sd.sc[0];
      s_ks[wave][16 + t] = sd.sc[1];
    }
    v8h pb[4];  // P' B operands, one per V scale block
    {
      v4f scv[8];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int r = 0; r < 4; ++r) scv[4 * s + r] = s_ks[wave][16 * s + 4 * g + r];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          pb[b][k] = (_Float16)(P[k] * __builtin_fminf(scv[k][b], kScaleCap));
    }

    // ---- PV: O^T[d, h] += V^T[d, tok] P'^T[tok, h] over the wave's 32 tokens
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) {
      const v2i raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(LDSP(v2i, (lat + v_off) ^ (16 * dt)));
      O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cvt8_f16(raw), pb[dt >> 3], O[dt], 0, 0, 0);
    }
  }

  // ---- epilogue
  l_run = xor_sum(l_run);  // lane (t, *) now holds head t's sum over this wave's tokens
  if constexpr (TG == 1) {
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    const float l2 = l_run > 0.0f ? m_run + __builtin_log2f(l_run) - kPShift : -INFINITY;
    if (h_ok) {
      if (split) {
        float* po = p.part_o + ((int64_t)unit * p.H + h) * kLat;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) *(v4f*)(po + 16 * dt + 4 * g) = O[dt] * inv;
        if (g == 0) p.part_lse[(int64_t)unit * p.H + h] = l2;
      } else {
        uint16_t* po = p.out + row * p.o_st + h * p.o_sh;
#pragma unroll
        for (int dt = 0; dt < 32; ++dt) {
          const v4f o = O[dt] * inv;
          const uint32_t w0 = f32_to_bf16_rne(o.x) | ((uint32_t)f32_to_bf16_rne(o.y) << 16);
          const uint32_t w1 = f32_to_bf16_rne(o.z) | ((uint32_t)f32_to_bf16_rne(o.w) << 16);
          *(v2i*)(po + 16 * dt + 4 * g) = v2i{(int)w0, (int)w1};
        }
        if (g == 0 && p.lse) p.lse[(int64_t)row * p.H + h] = l2 * kLn2;
      }
    }
  } else {
    // token groups of a head tile merge through LDS: weights 2^(m_own - M)
    if (g == 0) {
      s_m[wave][t] = m_run;
      s_l[wave][t] = l_run;
    }
    __syncthreads();  // every wave is done with the stage buffers
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < TG; ++k) M = fmax_(M, s_m[k * HT + ht][t]);
    const float w_own = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
    float* mrg = (float*)s_big;
    float* mine = mrg + ((tg * HT + ht) * 16 + t) * kMergeRow;
#pragma unroll
    for (int dt = 0; dt < 32; ++dt) *(v4f*)(mine + 16 * dt + 4 * g) = O[dt] * w_own;
    __syncthreads();
    constexpr int kDpw = kLat / TG;     // dims this wave reduces
    constexpr int kDpl = kDpw / 64;     // dims per lane (2 or 4)
    const int d0 = tg * kDpw + lane * kDpl;
    for (int hh = 0; hh < 16; ++hh) {
      const int hd = 16 * ht + hh;
      if (hd >= p.H) break;
      float Mh = -INFINITY;
#pragma unroll
      for (int k = 0; k < TG; ++k) Mh = fmax_(Mh, s_m[k * HT + ht][hh]);
      float L = 0.0f;
#pragma unroll
      for (int k = 0; k < TG; ++k) {
        const float mk = s_m[k * HT + ht][hh];
        if (mk != -INFINITY) L += s_l[k * HT + ht][hh] * __builtin_amdgcn_exp2f(mk - Mh);
      }
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      const float l2 = L > 0.0f ? Mh + __builtin_log2f(L) - kPShift : -INFINITY;
      float acc[kDpl];
#pragma unroll
      for (int e = 0; e < kDpl; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int k = 0; k < TG; ++k) {
        const float* src = mrg + ((k * HT + ht) * 16 + hh) * kMergeRow + d0;
#pragma unroll
        for (int e = 0; e < kDpl; ++e) acc[e] += src[e];
      }
      if (split) {
        float* po = p.part_o + ((int64_t)unit * p.H + hd) * kLat + d0;
#pragma unroll
        for (int e = 0; e < kDpl; ++e) po[e] = acc[e] * inv;
        if (tg == 0 && lane == 0) p.part_lse[(int64_t)unit * p.H + hd] = l2;
      } else {
        uint16_t* po = p.out + row * p.o_st + hd * p.o_sh + d0;
#pragma unroll
        for (int e = 0; e < kDpl; e += 2) {
          const uint32_t w = f32_to_bf16_rne(acc[e] * inv) | ((uint32_t)f32_to_bf16_rne(acc[e + 1] * inv) << 16);
          *(uint32_t*)(po + e) = w;
        }
        if (tg == 0 && lane == 0 && p.lse) p.lse[(int64_t)row * p.H + hd] = l2 * kLn2;
      }
    }
  }
}

// ---------------------------------------------------------------- combine

// LSE merge of a split row's chunks (K2-back page, stage_combine, without the
// sink): M = max_c lse2_c, w_c = 2^(lse2_c - M), out = sum w_c o_c / sum w_c.
__global__ __launch_bounds__(128) void smla_combine_kernel(CombineParams p) {
  int rank, h;
  xcd_unit(p.H, rank, h);
  if (rank >= p.T) return;
  const int row = p.order[rank];
  const int64_t u0 = (int64_t)row * p.S;
  float M = -INFINITY;
  for (int c = 0; c < p.S; ++c) M = fmax_(M, p.part_lse[(u0 + c) * p.H + h]);
  v4f acc = v4f{0, 0, 0, 0};
  float L = 0.0f;
  if (M != -INFINITY) {
    for (int c = 0; c < p.S; ++c) {
      const float lc = p.part_lse[(u0 + c) * p.H + h];
      if (lc == -INFINITY) continue;
      const float w = __builtin_amdgcn_exp2f(lc - M);
      L += w;
      acc += w * *(const v4f*)(p.part_o + ((u0 + c) * p.H + h) * kLat + 4 * threadIdx.x);
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  const v4f o = acc * inv;
  const uint32_t w0 = f32_to_bf16_rne(o.x) | ((uint32_t)f32_to_bf16_rne(o.y) << 16);
  const uint32_t w1 = f32_to_bf16_rne(o.z) | ((uint32_t)f32_to_bf16_rne(o.w) << 16);
  *(v2i*)(p.out + row * p.o_st + h * p.o_sh + 4 * threadIdx.x) = v2i{(int)w0, (int)w1};
  if (threadIdx.x == 0 && p.lse)
    p.lse[(int64_t)row * p.H + h] = L > 0.0f ? (M + __builtin_log2f(L)) * kLn2 : -INFINITY;
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

// ---------------------------------------------------------------- launchers

hipError_t launch_plan(const PlanParams& p, hipStream_t s) {
  const int blocks = (p.T + 3) / 4;
  hipLaunchKernelGGL(smla_plan_kernel, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

template <int HT, int TG>
static hipError_t launch_fwd_t(const FwdParams& p, hipStream_t s) {
  const int64_t blocks = xcd_grid(p.T, p.S);
  hipLaunchKernelGGL((smla_fwd_kernel<HT, TG>), dim3((unsigned)blocks), dim3(FwdCfg<HT, TG>::kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& p, hipStream_t s) {
  switch (head_tiles(p.H)) {
    case 1: return launch_fwd_t<1, 4>(p, s);
    case 2: return launch_fwd_t<2, 2>(p, s);
    case 3: return launch_fwd_t<3, 1>(p, s);
    case 4: return launch_fwd_t<4, 1>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const CombineParams& p, hipStream_t s) {
  const int64_t blocks = xcd_grid(p.T, p.H);
  hipLaunchKernelGGL(smla_combine_kernel, dim3((unsigned)blocks), dim3(128), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_decode_rows(const uint8_t* kv, int64_t n_kv, const int32_t* rows, int64_t n,
                              float* out, hipStream_t s) {
  hipLaunchKernelGGL(smla_decode_rows_kernel, dim3((unsigned)n), dim3(64), 0, s, kv, n_kv, rows, n, out);
  return hipGetLastError();
}

}  // namespace smla
