/*
 * smla.h -- C ABI of the sparse MLA forward library (libsmla.so) for MI355X
 * (gfx950, CDNA4).
 *
 * The operation (vLLM API page "vllm.models.kimi_k3.amd.ops.flydsl_sparse_mla_gfx950",
 * module docstring and the epilogue of build_sparse_mla_fp8ds_module): for each
 * query row r and head h, softmax attention of q[r, h, 0:576] over the KV
 * records listed in the row's CSR slice indices[indptr[r] .. indptr[r+1]),
 * where a record is decoded to K (576 values) and V (its first 512), logits are
 * scaled by sm_scale, out[r, h, 0:512] is the attention output and lse[r, h] the
 * natural-log log-sum-exp of the scaled logits.
 *
 * KV record, 656 bytes (same page, module docstring, "Record (656 B)"):
 *   bytes   0..511  512 e4m3 (OCP E4M3FN) latent codes
 *   bytes 512..527  4 little-endian f32 power-of-two scales; scale b applies to
 *                   latent values 128b .. 128b+127
 *   bytes 528..655  64 bf16 rope values
 *   K = [latent * scale, rope], V = latent * scale.
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are device memory the caller owns and keeps
 *     alive until the work queued on `stream` has finished; the library never
 *     frees or retains them.  `stream` is a hipStream_t (NULL = the null
 *     stream).  Work is queued asynchronously; no entry point synchronises
 *     the host unless stated.
 *   - The kernels run on the stream's device (the current device for the
 *     null stream), whatever device is current; every device pointer must be
 *     on that device.
 *   - Every entry point returns SMLA_OK (0) or a negative smla_status.  On a
 *     negative status nothing was queued, and sparse_mla_last_error() returns
 *     a message for the calling thread.
 *   - Element strides are in elements of the tensor's own type.
 */
#ifndef SMLA_H
#define SMLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SMLA_OK = 0,
  SMLA_EINVAL = -1,          /* malformed argument (null pointer, negative size, alignment, overflow) */
  SMLA_EUNSUPPORTED = -2,    /* well formed but outside what the kernels implement (e.g. heads > 64) */
  SMLA_EWORKSPACE = -3,      /* workspace missing or smaller than sparse_mla_workspace_bytes() */
  SMLA_EHIP = -4             /* a HIP runtime call failed; the message carries hipGetErrorString */
} smla_status;

/* Largest head count the kernels implement (they tile heads by 16; above
 * 64 heads a row's heads are processed in groups of 64). */
#define SMLA_MAX_HEADS 128

/*
 * sparse_mla_supported -- 1 if a forward with `num_heads` heads, QK head
 * dimension `head_dim_qk` and value dimension `dv` is implemented, else 0.
 * The record fixes head_dim_qk = 576 (512 latent + 64 rope) and dv = 512
 * (FlyDSL page, module docstring).  The FlyDSL page rejects head counts
 * outside [1, 16] (build_sparse_mla_fp8ds_module); this library accepts
 * [1, SMLA_MAX_HEADS].
 */
int sparse_mla_supported(int32_t num_heads, int32_t head_dim_qk, int32_t dv);

/*
 * sparse_mla_workspace_bytes -- device workspace a forward of T query rows,
 * H heads and nnz CSR entries needs on the current device (per-row tile
 * counts, the longest-first row order with each slot's unit descriptor and,
 * when rows are split, chunk partials).  Returns the byte count, or a negative smla_status for invalid
 * arguments; the size covers either has_invalid.  The workspace needs no
 * initialisation; it must not be shared by forwards that may run concurrently.
 */
int64_t sparse_mla_workspace_bytes(int32_t T, int32_t H, int64_t nnz);

/*
 * sparse_mla_split_for -- chunks per row (>= 1) a forward of T rows, H heads,
 * nnz entries and the given has_invalid uses on the current device: rows are
 * split, and the chunks merged by their log-sum-exp, when there are too few
 * rows to give every compute unit work; a padded batch (has_invalid) of about
 * one row per compute unit is also split in two, so that its longest rows
 * (queued first) can use two compute units.  Negative smla_status for invalid
 * arguments.
 */
int32_t sparse_mla_split_for(int32_t T, int32_t H, int64_t nnz, int32_t has_invalid);

/*
 * sparse_mla_fwd -- sparse MLA forward over fp8_ds_mla records.
 *
 *   q          device, bf16 [T, H, 576]: element (r, h, d) at
 *              q + r*q_stride_t + h*q_stride_h + d.  Dims 0..511 meet the
 *              latent, 512..575 the rope.  16-byte aligned, strides multiples of 8.
 *   kv         device, uint8 [n_kv, 656], rows contiguous, 16-byte aligned.
 *              Rows are addressed with 64-bit offsets, so the cache may exceed
 *              4 GiB.  Not bounds-checked (see preconditions).
 *   indptr     device, int32 [T + 1].  Row r's slice is
 *              indices[indptr[r] .. indptr[r+1]); a negative length is empty.
 *   indices    device, int32 [nnz] (may be NULL when nnz == 0).  Entries < 0
 *              mean "no key" and are ignored whatever has_invalid says.
 *              Index reads are bounded by nnz: a malformed indptr cannot read
 *              past the buffer (such positions read as index 0).
 *   sm_scale   logit scale (e.g. 1/sqrt(576)).
 *   has_invalid  nonzero: the caller pads slices with trailing entries < 0;
 *              tiles after the last entry >= 0 of a row are skipped (found by a
 *              scan of the slice, in the forward itself or in the plan kernel
 *              when there is one).  Zero: every slice position is scheduled.
 *              The result is the same either way.
 *   out        device, bf16 [T, H, 512] at out + r*o_stride_t + h*o_stride_h + d;
 *              16-byte aligned, strides multiples of 8.
 *   lse        device, f32 [T, H] contiguous, or NULL to skip it.  Natural log;
 *              -inf for a row with no key (whose out is all zero).
 *   workspace  device, >= sparse_mla_workspace_bytes(T, H, nnz) bytes (asked
 *              with the stream's device current: the split follows that
 *              device's compute units), 256-byte aligned.
 *
 * Preconditions the library cannot check (undefined results if broken, as on
 * the FlyDSL page, section "Preconditions the host cannot check"):
 *   - every per-128 scale is a positive power of two: the QK stage applies
 *     only the scale's exponent field (a mantissa or sign is dropped, and a
 *     zero scale acts as 2^-127, i.e. as a zero latent in practice), while the
 *     P.V stage uses the stored value;
 *   - every per-128 scale is <= 2^7: a larger one is clamped to 2^7 in the P.V
 *     product, which keeps the output finite but inexact;
 *   - every consumed index i satisfies 0 <= i < n_kv;
 *   - indptr is non-decreasing within [0, nnz] (violations are memory-safe but
 *     give unspecified rows).
 *
 * Returns SMLA_OK, or SMLA_EINVAL / SMLA_EUNSUPPORTED / SMLA_EWORKSPACE /
 * SMLA_EHIP with nothing queued (SMLA_EINVAL also when T is so large that a
 * launch would need 2^31 or more blocks: T * max(S * head groups, H) rounded
 * up, far beyond any q that fits in memory).  Queues on `stream`: a plan when there are
 * more (row, chunk, head group) units than compute units (a slice scan when has_invalid,
 * then a one-block longest-first sort of the rows; otherwise every unit
 * starts at once, rows run in their own order and each forward block scans
 * its own slice); the forward; and a combine when rows are split.  No host
 * sync, no allocation.
 * Deterministic for a fixed device and arguments.  nnz must be below
 * 2^30 - 4096 (index reads use 32-bit byte offsets).
 */
int sparse_mla_fwd(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                   const void* kv, int64_t n_kv,
                   const int32_t* indptr, const int32_t* indices, int64_t nnz,
                   int32_t T, int32_t H, float sm_scale, int32_t has_invalid,
                   void* out, int64_t o_stride_t, int64_t o_stride_h,
                   float* lse,
                   void* workspace, int64_t workspace_bytes,
                   void* stream);

/*
 * sparse_mla_fwd_noalloc -- sparse_mla_fwd without a workspace argument, for
 * callers that cannot allocate device memory: code being captured into a HIP
 * graph, tight serving loops, harnesses that forbid allocation.
 *
 * Every argument but the workspace, the semantics and the result are those of
 * sparse_mla_fwd (the same kernels on the same split).  The scratch that the
 * workspace would hold lives in a static device array of
 * SMLA_NOALLOC_SCRATCH_BYTES bytes: each device the library runs on holds its
 * own copy until the process ends.  The first call on a device looks its
 * address up (no allocation); no call allocates device or host memory.
 *
 * Calls on one device share that device's array and leave the last call's
 * contents in it (nothing in it needs to start at zero).  Calls that may
 * overlap on one device race on it: queue them on one stream, or use
 * sparse_mla_fwd with a workspace per stream.
 *
 * Returns SMLA_EWORKSPACE, with nothing queued, when the forward needs more
 * scratch than the array holds (sparse_mla_workspace_bytes(T, H, nnz) >
 * SMLA_NOALLOC_SCRATCH_BYTES: split partials of many long rows with many
 * heads); otherwise the statuses of sparse_mla_fwd.
 */
#define SMLA_NOALLOC_SCRATCH_BYTES (64LL << 20)
int sparse_mla_fwd_noalloc(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                           const void* kv, int64_t n_kv,
                           const int32_t* indptr, const int32_t* indices, int64_t nnz,
                           int32_t T, int32_t H, float sm_scale, int32_t has_invalid,
                           void* out, int64_t o_stride_t, int64_t o_stride_h,
                           float* lse, void* stream);

/*
 * smla_kv_pool -- one paged pool of 656-byte records (K2-back page of the
 * DeepSeek V4.1 AMD attention module, "key_rec": a key-table entry names a
 * slot of the window pool or of the compressed pool; a pool is a run of
 * pages).  Slot s of a pool is the record at
 *   base + (s / page_records) * page_stride + (s % page_records) * 656.
 *   base          device, page 0, 16-byte aligned; NULL: the pool is absent and
 *                 entries naming it are not keys.
 *   page_stride   bytes from one page to the next: a multiple of 16 and at
 *                 least page_records * 656 (a page may carry trailing bytes
 *                 that are never read).
 *   page_records  records per page, a power of two in [1, 2^30].
 */
typedef struct smla_kv_pool {
  const void* base;
  int64_t page_stride;
  int64_t page_records;
} smla_kv_pool;

/*
 * sparse_mla_fwd_paged -- sparse_mla_fwd over two paged pools, with an
 * optional per-head attention sink (K2-back page: "key_rec" for the entries,
 * "stage_combine" for the sink).
 *
 *   pools      host, smla_kv_pool[2]: pools[0] the window pool, pools[1] the
 *              compressed pool.  Read during the call only.
 *   indices    device, int32 [nnz]: -1 is no key; an entry e >= 0 is slot e
 *              of pools[0]; any other negative entry is slot (e & 0x7fffffff)
 *              of pools[1] (the slot with bit 31 set).  Entries naming an
 *              absent pool are no key.
 *   has_invalid  nonzero: slices may hold entries that are no key (-1, or of
 *              an absent pool); as in sparse_mla_fwd, trailing ones are skipped
 *              and the result is the same either way.
 *   sink       device, f32 [H] natural-log logits, or NULL for none.  Head h
 *              gains one more key of logit sink[h] (not scaled by sm_scale)
 *              and value 0: it joins the softmax maximum and sum but adds
 *              nothing to out.  A row with no key gets out = 0 and lse = sink[h]
 *              (-inf without a sink).  Finite or -inf values.
 * Every other argument, the workspace and the behaviour are those of
 * sparse_mla_fwd (with lse including the sink's term).  Preconditions the
 * library cannot check: every consumed slot lies inside its pool's
 * allocation, and the records meet sparse_mla_fwd's scale preconditions.
 * Returns SMLA_OK, or SMLA_EINVAL (also for a malformed pool descriptor) /
 * SMLA_EUNSUPPORTED / SMLA_EWORKSPACE / SMLA_EHIP with nothing queued.
 */
int sparse_mla_fwd_paged(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                         const smla_kv_pool* pools,
                         const int32_t* indptr, const int32_t* indices, int64_t nnz,
                         int32_t T, int32_t H, float sm_scale, int32_t has_invalid,
                         const float* sink,
                         void* out, int64_t o_stride_t, int64_t o_stride_h,
                         float* lse,
                         void* workspace, int64_t workspace_bytes,
                         void* stream);

/*
 * The DeepSeek V4.1 key record and its fused output epilogue (K2-back page:
 * "key_rec" for the layout, "stage_split" for the attention, "stage_combine"
 * for the merge, the sink and the epilogue).
 *
 * A key is 576 data bytes -- 448 e4m3 (OCP E4M3FN) "nope" values, then 64
 * bf16 rope values -- and 8 scale bytes, of which byte c (c < 7) is the E8M0
 * scale 2^(byte - 127) of nope dims 64c .. 64c+63.  K = [nope * scale, rope]
 * (512 dims) and V is the same 512 values.  Keys live in two paged pools
 * (smla_kv_pool, entries as in sparse_mla_fwd_paged): a page of R =
 * page_records keys holds their data (R x 576 bytes) and then their scale
 * words (R x 8 bytes), so key slot s is at
 *   data:  base + (s / R) * page_stride + (s % R) * 576
 *   scale: base + (s / R) * page_stride + R * 576 + (s % R) * 8,
 * with page_stride >= R * 584 and a multiple of 16.
 *
 * The output of row r, head h (the attention result over the keys, with the
 * sink folded in) is rounded to bf16, dims 448 + 2i and 448 + 2i + 1 (i < 32)
 * are rotated back by the inverse GPT-J rotation at the row's position
 * (e' = e cos_i + o sin_i, o' = o cos_i - e sin_i, cos_i = cos_sin[pos][i],
 * sin_i = cos_sin[pos][32 + i]), and each 32 dims are quantised to MXFP8:
 * E = floor(log2 amax) - 8 (at least -127; a zero block gives -127), the
 * scale byte E + 127, and the E4M3 codes of the values / 2^E clamped to
 * +-448, rounded to the nearest even.  (The pages name "vLLM's MXFP8"
 * without its rule; this is the OCP Microscaling v1.0 one.)
 */

/* Workspace a V4.1 forward needs (every row writes partials); [1, 16] heads. */
int64_t sparse_mla_v41_workspace_bytes(int32_t T, int32_t H, int64_t nnz);

/*
 * sparse_mla_fwd_v41 -- attention over V4.1 keys with the fused epilogue.
 *   q          device, bf16 [T, H, 512] (the rotated query) at q + r*q_stride_t
 *              + h*q_stride_h + d; 16-byte aligned, strides multiples of 8.
 *   pools      host, smla_kv_pool[2] (window pool, compressed pool), as above.
 *   indptr, indices, nnz, T, sm_scale, has_invalid, sink: as
 *              sparse_mla_fwd_paged.  H in [1, 16].
 *   pos        device, int32 [T]: each row's position (clamped to [0, n_pos)).
 *   cos_sin    device, f32 [n_pos, 64]: 32 cos, then 32 sin per position.
 *   xo         device, uint8 [T, H, 512] E4M3 codes, contiguous, 4-byte aligned.
 *   xo_scales  device, uint8 [T, H, 16] E8M0 bytes (dims 32j .. 32j+31).
 *   lse        device, f32 [T, H] natural log (sink included), or NULL.
 *   y_out      device, f32 [T, H, 512] or NULL: the values the MXFP8 step
 *              quantises (bf16-rounded output, rope dims rotated back), for
 *              checking the epilogue.
 *   workspace  >= sparse_mla_v41_workspace_bytes(T, H, nnz) bytes, 256-byte aligned.
 * Preconditions the library cannot check: consumed slots lie inside their
 * pool; scale bytes <= 134 (a scale above 2^7 is clamped to 2^7 in the P.V
 * stage); |rope values| < 2^15 (the partials are f16).
 * Queues the forward (partials) and the combine + epilogue on `stream` (and
 * the plan, as sparse_mla_fwd does).  Returns SMLA_OK, or a negative status
 * with nothing queued.
 */
int sparse_mla_fwd_v41(const void* q, int64_t q_stride_t, int64_t q_stride_h,
                       const smla_kv_pool* pools,
                       const int32_t* indptr, const int32_t* indices, int64_t nnz,
                       int32_t T, int32_t H, float sm_scale, int32_t has_invalid,
                       const float* sink, const int32_t* pos, const float* cos_sin, int32_t n_pos,
                       void* xo, void* xo_scales, float* lse, float* y_out,
                       void* workspace, int64_t workspace_bytes, void* stream);

/*
 * sparse_mla_mxfp8 -- test hook: the epilogue's MXFP8 quantiser (same device
 * code) on n f32 values y (n a multiple of 64): codes uint8 [n] (8-byte
 * aligned) and scales uint8 [n / 32], with the rule stated above.
 */
int sparse_mla_mxfp8(const float* y, int64_t n, void* codes, void* scales, void* stream);

/*
 * sparse_mla_qk_probe -- test hook: the QK dot products q . K (no sm_scale)
 * of the n records kv[rows[i]] (n a multiple of 16) against the 16 heads of
 * q (device bf16 [16, 576], contiguous), written to scores (device f32
 * [n, 16]).  It measures the QK stage on its own:
 *   mode 0  the forward's QK: K decoded exactly to bf16 with the record's
 *           power-of-two scale, bf16 MFMA 16x16x32, f32 accumulation;
 *   mode 1  the scaled fp8 MFMA 16x16x128 of the FlyDSL page (module
 *           docstring, "QK:"): K's e4m3 codes with the record scale as the
 *           E8M0 operand scale; q per head and 128-dim block split into an
 *           e4m3 hi part under scale s (the smallest power of two with
 *           amax / s <= 448) and an e4m3 lo part = 32 (q / s - hi) under s / 32;
 *   mode 2  mode 1 without the lo part;
 *   mode 3  mode 1 with lo = 16 (q / s - hi) under s / 16 (a top-binade hi's
 *           residual reaches 16, and 32 x 16 is past e4m3's 448).
 * Rope (64 dims) uses the bf16 MFMA in every mode.  Rows outside [0, n_kv)
 * read record 0.  Returns SMLA_EINVAL on bad arguments.
 */
int sparse_mla_qk_probe(const void* q, const void* kv, int64_t n_kv, const int32_t* rows, int64_t n,
                        int32_t mode, float* scores, void* stream);

/*
 * sparse_mla_decode_rows -- test hook: decode records rows[0..n) of kv to f32
 * out[n, 576] (latent * scale, then rope) exactly as the forward's QK stage
 * sees them (scale applied through its exponent field), cross-checked on the
 * device against the P.V stage's conversion for positive power-of-two scales
 * (a disagreement yields NaN).  A row index outside [0, n_kv) yields a row of
 * NaN.
 *   kv device uint8 [n_kv, 656]; rows device int32 [n]; out device f32 [n, 576].
 */
int sparse_mla_decode_rows(const void* kv, int64_t n_kv, const int32_t* rows, int64_t n,
                           float* out, void* stream);

/*
 * sparse_mla_cache_write -- write KV records in the fp8_ds_mla layout (the
 * step before the forward: vLLM's concat_and_cache_ds_mla writer, whose rule
 * the FlyDSL page states in its section "Preconditions the host cannot
 * check").  For token i with slots[i] in [0, n_kv), record slots[i] of kv
 * becomes:
 *   bytes   0..511  e4m3 (OCP E4M3FN) codes of latent[i, j] / scale[j / 128],
 *                   rounded to nearest, ties to even;
 *   bytes 512..527  the four f32 scales, scale[b] = pow2ceil(max(amax_b, 1e-4)
 *                   / 448) with amax_b the largest |latent[i, 128b .. 128b+127]|
 *                   (a power of two, so every record satisfies the forward's
 *                   preconditions whenever |latent| <= 57344);
 *   bytes 528..655  rope[i, 0..63] as bf16, copied.
 * Tokens with slots[i] < 0 (padding) or >= n_kv are skipped; no other byte of
 * kv changes.  Two tokens with the same slot race (either record may win).
 *
 *   latent  device, bf16 [n, 512] at latent + i*latent_stride + j; 16-byte
 *           aligned, latent_stride a multiple of 8 elements.  Finite values.
 *   rope    device, bf16 [n, 64] at rope + i*rope_stride + j; 8-byte aligned,
 *           rope_stride a multiple of 4 elements.
 *   slots   device, int64 [n], 8-byte aligned.
 *   kv      device, uint8 [n_kv, 656], rows contiguous, 16-byte aligned.
 * Returns SMLA_OK, or SMLA_EINVAL / SMLA_EHIP with nothing queued.  Queues one
 * kernel on `stream`; no host sync, no allocation.
 */
int sparse_mla_cache_write(const void* latent, int64_t latent_stride,
                           const void* rope, int64_t rope_stride,
                           const int64_t* slots, int64_t n,
                           void* kv, int64_t n_kv, void* stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* sparse_mla_last_error(void);

/*
 * sparse_mla_set_option -- tuning / test knobs, process-wide, not thread-safe
 * against concurrent forwards.  Names:
 *   "split"  chunks per row when rows are split (0 = automatic, 1 = never,
 *            2..SMLA_MAX_SPLIT forced); the workspace size accounts for it.
 *   "plan"   the plan kernels (has_invalid scan, longest-first order):
 *            0 = automatic (when units outnumber compute units), 1 = never
 *            (each forward block scans its own slice), 2 = always.
 *   "persist" with the plan and more units than compute units (for up to 16
 *            heads, at most twice as many), the kernels for up to 16 and for
 *            33 to 128 heads run a grid of one block per compute unit, each
 *            block taking several units in turn:
 *            0 = automatic, 1 = one unit per block always.  Results are the
 *            same either way.
 * Returns SMLA_OK or SMLA_EINVAL for an unknown name or value.
 */
#define SMLA_MAX_SPLIT 32
int sparse_mla_set_option(const char* name, int64_t value);

/*
 * Kernel timing for benchmarks.  sparse_mla_profile_begin(max_calls) makes the
 * following forwards (up to max_calls of them, on any stream) time each kernel
 * kind they queue with a HIP event pair attached to the kernel dispatches
 * themselves (hipExtLaunchKernel: start at the first dispatch's start, stop at
 * the last one's end, so queueing between launches is not counted);
 * sparse_mla_profile_end() waits for
 * those events, writes the summed device time in milliseconds and the launch
 * count of each kernel kind (0 plan, 1 forward, 2 combine, 3 cache writer) to
 * ms[SMLA_PROFILE_KINDS] and launches[SMLA_PROFILE_KINDS], and stops
 * recording.  Calls of sparse_mla_cache_write are recorded too.  Creates and destroys events on the host
 * only; no device memory is allocated.
 */
#define SMLA_PROFILE_KINDS 4
int sparse_mla_profile_begin(int32_t max_calls);
int sparse_mla_profile_end(double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* SMLA_H */
