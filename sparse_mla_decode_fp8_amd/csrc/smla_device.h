// Device-side helpers shared by the forward kernels (smla_kernels.hip,
// smla_wide.hip): vector types, LDS and DMA access, exact e4m3 conversions,
// the XCD-aware unit mapping, key addressing, the tile count of a unit and
// the final softmax normalisation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "smla_internal.h"

namespace smla {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));

#define LDSP(T, off) ((__attribute__((address_space(3))) T*)(uintptr_t)(off))
#define GLBP(T, addr) ((const __attribute__((address_space(1))) T*)(uintptr_t)(addr))

constexpr int kLat = 512;
constexpr int kScaleOff = 512;
constexpr int kRopeOff = 528;
constexpr float kScaleCap = 128.0f;  // 2^7: P' = P * scale <= 2^15 fits f16
constexpr float kLn2 = 0.693147180559945309f;

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
// 4 bytes per lane through a bounded buffer descriptor (reads past its size
// return 0) into LDS at lds_base + 4*lane.
__device__ __forceinline__ void buf_dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :: "v"(voffset), "s"(rsrc), "s"(lds_base) : "memory", "m0");
}
#pragma clang diagnostic pop

// vmcnt(0) only (expcnt, lgkmcnt left at their maxima), through the intrinsic
// so the compiler's own wait tracking knows every load has completed here.
__device__ __forceinline__ void wait_vm_all() {
  __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ float fmax_(float a, float b) { return __builtin_fmaxf(a, b); }

// Max / sum over the four lanes t, t+16, t+32, t+48.  v_permlane16_swap
// exchanges the odd 16-lane rows of its first operand with the even rows of
// its second; given two copies of one value, every lane ends with its own
// value in one result and that of lane ^ 16 in the other.  v_permlane32_swap
// does the same for the two 32-lane halves (lane ^ 32).  Both are VALU
// operations, with no LDS round trip.  Max and sum of the two results are
// symmetric, so partner lanes agree bit for bit.
// The two results pass through an empty asm before they are used as floats:
// the ROCm 7.2 compiler otherwise folds the second result of the swap into
// the first when both feed one float operation (f(r[0]) + f(r[1]) is emitted
// as r[0] + r[0]).
__device__ __forceinline__ float2 swap_pair(__attribute__((ext_vector_type(2))) uint32_t r) {
  uint32_t a = r[0], b = r[1];
  asm volatile("" : "+v"(a), "+v"(b));
  return float2{__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)};
}
__device__ __forceinline__ float2 swap16(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return swap_pair(__builtin_amdgcn_permlane16_swap(u, u, false, false));
}
__device__ __forceinline__ float2 swap32(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  return swap_pair(__builtin_amdgcn_permlane32_swap(u, u, false, false));
}
__device__ __forceinline__ float xor_max(float v) {
  // the maxima in asm: on values the compiler cannot see it would first
  // canonicalise each operand (two more dependent instructions per step)
  float2 a = swap16(v);
  asm("v_max_f32 %0, %1, %2" : "=v"(v) : "v"(a.x), "v"(a.y));
  a = swap32(v);
  asm("v_max_f32 %0, %1, %2" : "=v"(v) : "v"(a.x), "v"(a.y));
  return v;
}
__device__ __forceinline__ float xor_sum(float v) {
  const float2 a = swap16(v);
  const float2 b = swap32(a.x + a.y);
  return b.x + b.y;
}

// Two f32 to two bf16, rounded to nearest even (one v_cvt_pk_bf16_f32; NaN
// stays NaN, overflow rounds to infinity), packed lo | hi << 16.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2bf));
}
// Four f32 to four packed bf16 (two words).
__device__ __forceinline__ v2i pack_bf16x4(v4f a) { return v2i{(int)pack_bf16x2(a.x, a.y), (int)pack_bf16x2(a.z, a.w)}; }
// An f32 rounded to bf16 (nearest even) and widened back to f32.
__device__ __forceinline__ float round_bf16(float f) { return __builtin_bit_cast(float, pack_bf16x2(f, 0.0f) << 16); }

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


// Split partials of the output are stored as f16: a normalised partial is a
// convex combination of V values, |V| <= 448 * 2^7 = 57344, so it fits f16's
// range, and its 11-bit precision is finer than the bf16 of the result.
//
// Partial layout (the workspace's own): within each 64-dim block of a head,
// the 4-dim pieces are stored in the order the MFMA accumulators hold them
// per lane: dims 16 dt + 4 g + [0..3] at position 16 g + 4 dt + [0..3].  A
// lane's 16 dims are then contiguous (32 B), and the combine, which reads
// position 4x .. 4x+3 in thread x, maps it back with part_dim().
__device__ __forceinline__ int part_dim(int pos) {  // dim held at a partial position
  return (pos & ~63) | (((pos >> 2) & 3) << 4) | (((pos >> 4) & 3) << 2) | (pos & 3);
}
// One lane's four accumulator pieces (dims 16 dt + 4 g + [0..3], dt = 0..3) of
// one head, normalised by `scale`, as f16 at block + 16 g.  Nontemporal: the
// combine reads the partials once, later, and nothing dirty is left in L2 for
// the end-of-kernel write-back.
__device__ __forceinline__ void st_part16(uint16_t* block, int g, const v4f o[4], float scale) {
  typedef _Float16 v8hh __attribute__((ext_vector_type(8)));
  v8hh a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = (_Float16)(o[0][i] * scale);
    a[4 + i] = (_Float16)(o[1][i] * scale);
    b[i] = (_Float16)(o[2][i] * scale);
    b[4 + i] = (_Float16)(o[3][i] * scale);
  }
  __builtin_nontemporal_store(a, (v8hh*)(block + 16 * g));
  __builtin_nontemporal_store(b, (v8hh*)(block + 16 * g + 8));
}
__device__ __forceinline__ v4f half4_to_f32(v2i raw) {
  const v4h hv = __builtin_bit_cast(v4h, raw);
  return v4f{(float)hv.x, (float)hv.y, (float)hv.z, (float)hv.w};
}

// XCD-aware unit mapping: block b runs on XCD b % 8; rows of rank r go to XCD
// r % 8 and the `per_row` blocks of a row are consecutive on that XCD.  A
// persistent block maps the virtual blocks b it runs (b, b + grid, ..., with
// the grid a multiple of 8, so all on its own XCD) the same way.
__device__ __forceinline__ void xcd_unit_at(int b, int per_row, int& rank, int& sub) {
  const int i = b >> 3;
  rank = (b & 7) + 8 * (i / per_row);
  sub = i % per_row;
}
__device__ __forceinline__ void xcd_unit(int per_row, int& rank, int& sub) {
  xcd_unit_at(blockIdx.x, per_row, rank, sub);
}

// Unit mapping of the split forward.  A row's keys in chunk order cover the
// record index range in order when its slice is sorted, so chunk c of every
// row touches about the same records at about the same time; putting those
// units on the same XCDs lets that XCD's L2 serve the records several rows
// share instead of fetching them once per row.  With `ranged`: S dividing 8,
// chunk c runs on XCDs [c 8/S, (c+1) 8/S) (rows spread over that group);
// S = 16 or 32, chunk c on XCD c mod 8.  Otherwise all chunks of a row run on
// one XCD (xcd_unit).  `ranged` is set only when every unit gets a CU of its
// own (no longest-first plan): with more units than CUs, the chunks of ragged
// rows differ in length, and grouping them by chunk would load some XCDs more
// than others.  The launch grid is fwd_grid(T, S, ranged).
__device__ __forceinline__ void fwd_unit(int S, bool ranged, int& rank, int& chunk) {
  const int x = blockIdx.x & 7;
  const int i = blockIdx.x >> 3;
  if (ranged && (S == 2 || S == 4 || S == 8)) {
    const int G = 8 / S;  // XCDs per chunk
    chunk = x / G;
    rank = (x % G) + G * i;
  } else if (ranged && (S == 16 || S == 32)) {
    const int k = S >> 3;  // chunks of a row on one XCD
    chunk = x + 8 * (i % k);
    rank = i / k;
  } else {
    xcd_unit(S, rank, chunk);
  }
}

// Record address of an index entry that is a key (KeyMode::valid).
__device__ __forceinline__ const uint8_t* key_addr(const FwdParams& p, int e) {
  if (!p.km.paged) return p.kv + (int64_t)e * kRecordBytes;
  // selects, not a dynamic index into the kernel argument (that would copy
  // the whole argument to scratch memory)
  const bool c = e < 0;
  const uint32_t slot = (uint32_t)e & 0x7FFFFFFFu;
  const uint32_t sh = (uint32_t)(c ? p.pool_shift[1] : p.pool_shift[0]);
  const uint8_t* const base = c ? p.pool[1] : p.pool[0];
  const int64_t stride = c ? p.pool_stride[1] : p.pool_stride[0];
  return base + (int64_t)(slot >> sh) * stride + (int64_t)(slot & ((1u << sh) - 1u)) * kRecordBytes;
}

// Tiles of a row from its effective length.
__device__ __forceinline__ int tiles_of(int len, int tile) { return (len + tile - 1) / tile; }

// Tiles of row `row` for a forward block of NT threads: the plan's count when
// there is a plan; with has_invalid and no plan, 1 + the last slice position
// whose entry is >= 0, found by every thread of the block (bounded index
// reads, one round of NT x 4 entries per pass) and a block-wide max through
// `red` (NT / 64 ints of LDS); otherwise the slice length.
template <int NT>
__device__ __forceinline__ int unit_tiles(const FwdParams& p, int row, int beg, int len, int tile, int* red) {
  if (p.row_tiles) return p.row_tiles[row];
  if (!p.scan) return tiles_of(len, tile);
  const __amdgpu_buffer_rsrc_t r = idx_rsrc(p.indices, p.idx_bytes);
  const int tid = threadIdx.x;
  int lastp = 0;
  for (int base = 0; base < len; base += 4 * NT) {
    int v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = load_idx(r, (uint32_t)(beg + base + NT * j + tid) * 4u);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int pos = base + NT * j + tid;
      if (pos < len && p.km.valid(v[j])) lastp = max(lastp, pos + 1);
    }
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) lastp = max(lastp, __shfl_xor(lastp, sh));
  if ((tid & 63) == 0) red[tid >> 6] = lastp;
  __syncthreads();
  int m = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) m = max(m, red[k]);
  return tiles_of(m, tile);
}

// s_waitcnt immediates (gfx9 layout: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14)
constexpr int waitcnt_vm(int n) { return (n & 0xF) | (0x7 << 4) | (0xF << 8) | (((n >> 4) & 0x3) << 14); }
constexpr int kWaitLgkm0 = 0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14);

// vmcnt waits with a compile-time count
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(N));
}

// 16 bytes from global memory into registers, issued from asm: the compiler
// does not count it, so it never inserts a wait for it; the kernel waits with
// explicit vmcnt counts and then pins the registers .
__device__ __forceinline__ void gload16(v4f& dst, uint64_t addr) {
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(dst) : "v"(addr) : "memory");
}
__device__ __forceinline__ void gload16(v4i& dst, uint64_t addr) {
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(dst) : "v"(addr) : "memory");
}

constexpr int kSideTok = 144;       // scales (16 B) + rope (128 B) of a record
constexpr int kSideChunks = 9;
constexpr float kShift = 4.0f;      // P = exp2(x - m_ref + 4)
constexpr float kTau = 4.0f;        // m_ref moves only when a head's max exceeds it by > 4

// A head's final normalisation.  l is its softmax sum of P = 2^(x - m + kShift)
// (m in log2 units), sink2 its sink logit in log2 units (-inf: none; the sink
// is one more key whose value is 0, K2-back page, stage_combine).  Returns the
// factor that turns the accumulated O into the output, and the lse in log2
// units.  Without a sink this is 1 / l and m - kShift + log2 l.
struct Norm {
  float scale, lse2;
};
__device__ __forceinline__ Norm finish_norm(float l, float m, float sink2) {
  const float mo = l > 0.0f ? m - kShift : -INFINITY;
  const float mm = fmax_(mo, sink2);
  if (mm == -INFINITY) return Norm{0.0f, -INFINITY};
  const float a = l > 0.0f ? __builtin_amdgcn_exp2f(mo - mm) : 0.0f;
  const float L = l * a + __builtin_amdgcn_exp2f(sink2 - mm);
  // L >= 1: a non-empty row's largest weight is at least 2^kShift (the lazy
  // reference never exceeds the running max), and a dominating sink adds 1.
  // So the hardware reciprocal and log2 (about 1 ulp, no denormal handling
  // needed) serve; the result is rounded to f16 or bf16 after.
  return Norm{a * __builtin_amdgcn_rcpf(L), mm + __builtin_amdgcn_logf(L)};
}
__device__ __forceinline__ float sink_log2(const float* sink, int h) {
  return sink ? sink[h] * 1.4426950408889634f : -INFINITY;
}

}  // namespace smla
