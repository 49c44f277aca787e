// Test hook: the QK scores of 16-token groups, computed two ways.
//
// The FlyDSL page (module docstring, "QK:" and the q prologue helpers) does the
// latent part of QK on gfx950's scaled fp8 MFMA: K's e4m3 codes enter with the
// record's power-of-two scale as the E8M0 operand scale, and q, per head and
// 128-dim block, is split into an e4m3 "hi" part under an E8M0 scale s and an
// e4m3 "lo" part holding 32 x the residual under scale s - 5; rope stays on a
// bf16 MFMA.  This library's forward instead dequantises K exactly to bf16 and
// uses the bf16 MFMA.  The hook computes both, on the same 16-token tile
// layout, so a test can measure each against fp64 scores.
//   mode 0: the forward's QK (K -> bf16 by v_cvt_scalef32_pk_bf16_fp8 with the
//           record scale, bf16 MFMA 16x16x32, f32 accumulation);
//   mode 1: scaled fp8 MFMA 16x16x128 with the q hi/lo split;
//   mode 2: the same with the hi part only;
//   mode 3: hi/lo with lo = 16 x the residual under scale s - 4 (the residual
//           of a top-binade hi reaches half its 32-unit step, and 32 x 16 =
//           512 is past e4m3's 448).
// Rope is the bf16 MFMA in every mode.  Output: the raw dot products q . K
// (no sm_scale), scores[token][head] for 16 heads.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_device.h"

namespace smla {

typedef int v8i __attribute__((ext_vector_type(8)));

// E8M0 exponent byte of a power-of-two f32 scale (its biased exponent field).
__device__ __forceinline__ int e8m0_of(float sc) { return (int)((__builtin_bit_cast(uint32_t, sc) >> 23) & 0xFF); }

// One wave per 16 tokens: lane (t, g) = (lane & 15, lane >> 4).
__global__ __launch_bounds__(64) void smla_qk_probe_kernel(const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv,
                                                           int64_t n_kv, const int32_t* __restrict__ rows, int mode,
                                                           float* __restrict__ scores) {
  const int lane = threadIdx.x;
  const int t = lane & 15;
  const int g = lane >> 4;
  int r = rows[blockIdx.x * 16 + t];
  r = (r < 0 || r >= n_kv) ? 0 : r;  // the caller passes valid rows; stay in bounds regardless
  const uint8_t* rec = kv + (int64_t)r * kRecordBytes;
  const uint16_t* qh = q + t * 576;  // head t (B column t)
  const v4f ksc = *(const v4f*)(rec + kScaleOff);

  v4f acc = v4f{0, 0, 0, 0};
  // rope (both modes): K-step i covers dims 512 + 32 i + 8 g + [0..7]
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const v8bf kr = __builtin_bit_cast(v8bf, *(const v4i*)(rec + kRopeOff + 64 * i + 16 * g));
    const v8bf qr = __builtin_bit_cast(v8bf, *(const v4i*)(qh + kLat + 32 * i + 8 * g));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr, qr, acc, 0, 0, 0);
  }
  if (mode == 0) {
    // the forward's latent QK: K-step pair m covers dims 64 m + 16 g + [0..15]
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const v4i kw = *(const v4i*)(rec + 64 * m + 16 * g);
      const float sc = ksc[m >> 1];
      v2bf a0, a1, a2, a3, b0, b1, b2, b3;
      cvt4_bf16(kw.x, sc, a0, a1);
      cvt4_bf16(kw.y, sc, a2, a3);
      cvt4_bf16(kw.z, sc, b0, b1);
      cvt4_bf16(kw.w, sc, b2, b3);
      const v8bf ka = {a0.x, a0.y, a1.x, a1.y, a2.x, a2.y, a3.x, a3.y};
      const v8bf kb = {b0.x, b0.y, b1.x, b1.y, b2.x, b2.y, b3.x, b3.y};
      const v8bf qa = __builtin_bit_cast(v8bf, *(const v4i*)(qh + 64 * m + 16 * g));
      const v8bf qb = __builtin_bit_cast(v8bf, *(const v4i*)(qh + 64 * m + 16 * g + 8));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qa, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb, acc, 0, 0, 0);
    }
  } else {
    // scaled fp8: block b, lane (t, g) holds K elements 32 g .. 32 g + 31 of
    // token t (A) and of head t (B); every lane of a row or column supplies
    // that row's or column's scale byte for the block.
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const v4i k0 = *(const v4i*)(rec + 128 * b + 32 * g);
      const v4i k1 = *(const v4i*)(rec + 128 * b + 32 * g + 16);
      const v8i ka = v8i{k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
      const int sa = e8m0_of(ksc[b]);
      float x[32];
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        x[j] = __builtin_bit_cast(float, (uint32_t)qh[128 * b + 32 * g + j] << 16);
        amax = fmax_(amax, __builtin_fabsf(x[j]));
      }
      amax = fmax_(amax, __shfl_xor(amax, 16));
      amax = fmax_(amax, __shfl_xor(amax, 32));
      // s: the smallest power of two with amax / s <= 448 (as the record
      // writer's rule), as an E8M0 byte; x' = x / s
      const uint32_t vb = __builtin_bit_cast(uint32_t, amax / 448.0f);
      const uint32_t pb = (vb & 0x007FFFFFu) ? (vb & 0x7F800000u) + 0x00800000u : vb;
      int sb = (int)(pb >> 23);
      sb = sb < 6 ? 6 : (sb > 253 ? 253 : sb);  // keep s and s - 5 normal E8M0 bytes
      const float inv = __builtin_bit_cast(float, (uint32_t)(254 - sb) << 23);  // 2^(127 - s)
      int hw[8], lw[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float y0 = x[4 * d] * inv, y1 = x[4 * d + 1] * inv, y2 = x[4 * d + 2] * inv, y3 = x[4 * d + 3] * inv;
        int h = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
        h = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, h, true);
        const float r0 = y0 - __builtin_amdgcn_cvt_f32_fp8(h, 0), r1 = y1 - __builtin_amdgcn_cvt_f32_fp8(h, 1);
        const float r2 = y2 - __builtin_amdgcn_cvt_f32_fp8(h, 2), r3 = y3 - __builtin_amdgcn_cvt_f32_fp8(h, 3);
        const float f = mode == 3 ? 16.0f : 32.0f;
        int l = __builtin_amdgcn_cvt_pk_fp8_f32(f * r0, f * r1, 0, false);
        l = __builtin_amdgcn_cvt_pk_fp8_f32(f * r2, f * r3, l, true);
        hw[d] = h;
        lw[d] = l;
      }
      const v8i qhi = v8i{hw[0], hw[1], hw[2], hw[3], hw[4], hw[5], hw[6], hw[7]};
      const v8i qlo = v8i{lw[0], lw[1], lw[2], lw[3], lw[4], lw[5], lw[6], lw[7]};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qhi, acc, 0, 0, 0, sa, 0, sb);
      if (mode != 2)
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qlo, acc, 0, 0, 0, sa, 0, mode == 3 ? sb - 4 : sb - 5);
    }
  }
  // C layout: lane (t, g) holds tokens 4 g + i of head t
#pragma unroll
  for (int i = 0; i < 4; ++i) scores[(blockIdx.x * 16 + 4 * g + i) * 16 + t] = acc[i];
}

hipError_t launch_qk_probe(const uint16_t* q, const uint8_t* kv, int64_t n_kv, const int32_t* rows, int64_t n,
                           int mode, float* scores, hipStream_t s) {
  hipLaunchKernelGGL(smla_qk_probe_kernel, dim3((unsigned)(n / 16)), dim3(64), 0, s, q, kv, n_kv, rows, mode, scores);
  return hipGetLastError();
}

}  // namespace smla
