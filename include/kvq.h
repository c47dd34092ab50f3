/*
 * kvq.h -- C ABI of the MI355X int4 KV-cache quantizer (libkvq.so).
 *
 * The method ("When Quantization Is Free: An int4 KV Cache That Outruns fp16
 * on Apple Silicon", M. A. Bergach, arXiv 2605.05699): every head vector of D
 * channels is rotated by a sign-randomized FFT (SRFT), or optionally by a
 * sign-randomized Walsh-Hadamard transform (SRHT), rescaled per channel by
 * lambda, split into groups of 32 channels that each get one fp16 abs-max
 * scale, and rounded to signed int4 codes packed two per byte.  The read side
 * undoes it: unpack, rescale, inverse rotation -- alone (kvq_decode) or fused
 * into decode-step attention (kvq_attn_decode).
 *
 * Sources, by page and section:
 *   [abstract]  the paper's abstract (paperdance.org and mlsanity.com pages):
 *               the fused pipeline, SRFT vs SRHT, the HuggingFace Cache role;
 *   [M1]        gist.science explainer, "Methodik" 1: SRFT(x) =
 *               pack(F . diag(s) . x), F the unitary DFT, s fixed random signs;
 *   [M2]        same page, "Methodik" 2: load and sign, log2(d/2) FFT passes,
 *               pack, per-channel lambda, per-group abs-max, round to int4,
 *               two nibbles per byte;
 *   [M3]        same page, "Methodik" 3: per-channel plus per-group scaling;
 *   [Mem]       same page, "Speichereffizienz": 3.0x-3.56x compression, i.e.
 *               int4 codes plus one fp16 scale per 32 channels.
 *
 * Conventions fixed here (the pages leave them open):
 *   - pairing: z_k = x[2k] + i x[2k+1], k < D/2; one sign per pair (SRFT) or
 *     per channel (SRHT); forward DFT kernel exp(-2 pi i k m / (D/2)) scaled by
 *     (D/2)^-1/2; the output Z_m is unpaired to channels 2m (real) and 2m+1
 *     (imaginary).  SRHT: y = D^-1/2 H_D (s . x), H_D in Sylvester order.
 *   - signs: bit i of the SplitMix64 stream seeded with the plan seed (bit
 *     i mod 64 of output i / 64), sign = 1 - 2 bit.
 *   - group g = output channels [32 g, 32 g + 32); scale = fp16(absmax / 7)
 *     (the fp32 quotient of the fp32 abs-max, rounded to nearest even to
 *     fp16, subnormals kept); code = clamp(rint_even(w /
 *     scale), -8, 7), 0 where scale == 0; nibble = code + 8, channel 2m in
 *     the low nibble of byte m.
 *   - variants (kvq_plan_create_ex): groups of G = 16 channels ([M3] uses
 *     groups of 16), and int8 codes ([M2] rounds to signed int4 or int8):
 *     scale = fp16(absmax / 127), code = clamp(rint_even(w / scale), -128,
 *     127), stored as one two's-complement byte per channel, in channel
 *     order.  A token's codes take D * bits / 8 bytes, its scales D / G fp16.
 *
 * Memory: every tensor pointer is a DEVICE pointer owned by the caller.  No
 * entry point allocates, frees or synchronizes; kernels are enqueued on the
 * caller's stream (a hipStream_t passed as void*, NULL = the default stream)
 * and device faults surface at the caller's next synchronization.  fp16 values
 * are passed as uint16_t bit patterns.  Strides are in elements, non-negative,
 * and every element a call reaches must lie within 2^62 elements of its base
 * pointer (KVQ_ERR_INVALID otherwise); byte offsets past 2^32 are supported.
 *
 * Errors: every argument check runs on the host before anything is enqueued;
 * a failing call has no side effects and returns a kvq_status other than
 * KVQ_OK, with a detail string from kvq_last_error() (per thread).  A launch
 * failure reported by the HIP runtime returns KVQ_ERR_HIP.  No C++ exception
 * crosses this interface.
 *
 * Concurrency: calls on different streams may run concurrently when their
 * outputs and workspaces do not overlap.  Inputs must not alias outputs.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = 1,      /* bad value: null pointer, size, stride, range */
  KVQ_ERR_UNSUPPORTED = 2,  /* valid but not built: D, G or rotation */
  KVQ_ERR_ALIGN = 3,        /* a pointer or row is not 16-byte aligned */
  KVQ_ERR_WORKSPACE = 4,    /* workspace missing or too small */
  KVQ_ERR_HIP = 5           /* the HIP runtime reported a launch error */
} kvq_status;

typedef enum {
  KVQ_SRFT = 0,             /* sign-randomized FFT [M1] */
  KVQ_SRHT = 1,             /* sign-randomized Walsh-Hadamard [abstract] */
  KVQ_IDENTITY = 2          /* no rotation: exercises the quantizer alone */
} kvq_rotation;

typedef enum { KVQ_F16 = 0, KVQ_F32 = 1 } kvq_dtype;

typedef struct kvq_plan kvq_plan;   /* opaque, immutable after creation */

/* Version string of the library build. */
const char* kvq_version(void);

/* Name of a status code; never NULL. */
const char* kvq_strerror(kvq_status s);

/* Detail of the last failed call on this thread ("" if none). */
const char* kvq_last_error(void);

/* Create a plan: head dimension D, group size G (32) and the rotation, with
 * the sign vector drawn from SplitMix64(seed) [M1].  Pure host work: no GPU
 * call.  *out receives a plan the caller releases with kvq_plan_destroy.
 * D = 128 or 256 take every rotation.  D = 96 and 80 (head sizes that are
 * not powers of two, where the DFT is factored over radices 2, 3, 4 and 5;
 * [abstract]: the SRFT is chosen because it has mixed-radix sizes) take
 * KVQ_SRFT and KVQ_IDENTITY; KVQ_SRHT needs a power of two.  G must divide
 * D (D = 80: G = 16).  Other values: KVQ_ERR_UNSUPPORTED. */
kvq_status kvq_plan_create(int32_t D, int32_t G, kvq_rotation rotation, uint64_t seed,
                           kvq_plan** out);

/* Create a plan with a code width and group size: bits = 4 (int4 nibbles) or
 * 8 (int8 bytes), G = 32 or 16 (dividing D); otherwise as kvq_plan_create,
 * which is this call with bits = 4.  KVQ_ERR_UNSUPPORTED for other widths or
 * groups. */
kvq_status kvq_plan_create_ex(int32_t D, int32_t G, int32_t bits, kvq_rotation rotation, uint64_t seed,
                              kvq_plan** out);

/* Plan options (bits of kvq_plan_create_opt's options). */
typedef enum {
  /* D = 128 SRFT: kvq_encode and kvq_rotate take the 64-point DFT on the
   * matrix cores, factored as 8 x 8 (the explainer's "Begruendung" for the
   * SRFT and its AMX path, "Methodik" 1 and 4: DFTs as small dense matrix
   * products).  Same codes and scales up to the boundary cases of a
   * different fp32 rounding order; decode and attention are unchanged. */
  KVQ_OPT_MFMA_ROTATION = 1
} kvq_option;

/* Create a plan with options: kvq_plan_create_ex plus a set of kvq_option
 * bits (0 = none).  KVQ_ERR_INVALID for unknown bits, KVQ_ERR_UNSUPPORTED
 * for an option the plan's D or rotation has no kernel for. */
kvq_status kvq_plan_create_opt(int32_t D, int32_t G, int32_t bits, kvq_rotation rotation, uint64_t seed,
                               uint32_t options, kvq_plan** out);

/* Read back a plan's option bits. */
kvq_status kvq_plan_options(const kvq_plan* plan, uint32_t* options);

/* Release a plan (NULL is a no-op).  Work already enqueued does not use the
 * plan object: its constants travel with each launch. */
void kvq_plan_destroy(kvq_plan* plan);

/* Copy the plan's sign vector to host memory: n = D/2 entries for SRFT, D for
 * SRHT, 0 for IDENTITY; each entry is +1 or -1.  n must equal that count. */
kvq_status kvq_plan_signs(const kvq_plan* plan, int8_t* host_signs, int64_t n);

/* Read back D, G and the rotation of a plan (any output may be NULL). */
kvq_status kvq_plan_info(const kvq_plan* plan, int32_t* D, int32_t* G, int32_t* rotation);

/* The same with the code width (4 or 8); any output may be NULL. */
kvq_status kvq_plan_info_ex(const kvq_plan* plan, int32_t* D, int32_t* G, int32_t* bits, int32_t* rotation);

/* Encode [M2]: for b < B, h < H, t < T rotate x[b,h,t,:] (fp16, element
 * (b,h,t,j) at x + b*x_sb + h*x_sh + t*x_st + j; each row 16-byte aligned),
 * multiply by lambda[b*lambda_sb + h*D + j] (fp32; lambda_sb = 0 shares one
 * [H,D] table across the batch), quantize per group and write token t0 + t of
 *   codes  uint8 [B, H, Tcap, D*bits/8]  (dense, 16-byte aligned; D/2 bytes
 *                                         for int4)
 *   scales fp16  [B, H, Tcap, D/G]       (dense; 16-byte aligned at D = 256
 *                                         and at D = 128 with G = 16, else
 *                                         8-byte aligned).
 * Requires 0 <= t0, t0 + T <= Tcap and a token stride x_st below 2^28
 * elements (else KVQ_ERR_INVALID).  B, H or T of 0 is a no-op.  The caller
 * owns every buffer; nothing is allocated or synchronized. */
kvq_status kvq_encode(const kvq_plan* plan, const uint16_t* x, int64_t B, int64_t H, int64_t T,
                      int64_t x_sb, int64_t x_sh, int64_t x_st,
                      const float* lambda, int64_t lambda_sb,
                      uint8_t* codes, uint16_t* scales, int64_t Tcap, int64_t t0,
                      void* stream);

/* Decode, the read side of [M1]/[M2] (the inverse of kvq_encode up to
 * quantization; R is orthogonal, so its inverse is R^T [M1]): for tokens
 * t0 .. t0+T-1 of codes/scales [B,H,Tcap,...] compute
 *   x^[j] = (R^T ( (q . scale) / lambda ))[j]
 * and write it to y (fp16 rounded to nearest even, or fp32) at
 * y + b*y_sb + h*y_sh + t*y_st + j; fp16 rows must be 16-byte aligned, fp32
 * rows 8-byte aligned.  At D = 128 and 256 lambda must be 16-byte aligned
 * with lambda_sb a multiple of 4, and scales aligned as for kvq_encode.
 * Requires 0 <= t0, t0 + T <= Tcap and y_st below 2^28 elements; B, H or T
 * of 0 is a no-op. */
kvq_status kvq_decode(const kvq_plan* plan, const uint8_t* codes, const uint16_t* scales,
                      int64_t B, int64_t H, int64_t Tcap, int64_t t0, int64_t T,
                      const float* lambda, int64_t lambda_sb,
                      void* y, kvq_dtype y_dtype, int64_t y_sb, int64_t y_sh, int64_t y_st,
                      void* stream);

/* Rotate only, [M1] followed by the lambda rescale of [M2] (a test hook
 * running the encoder's own transform): w[b,h,t,:] = lambda . (R x[b,h,t,:])
 * in fp32, w dense [B, H, T, D] and 16-byte aligned; x and lambda as for
 * kvq_encode. */
kvq_status kvq_rotate(const kvq_plan* plan, const uint16_t* x, int64_t B, int64_t H, int64_t T,
                      int64_t x_sb, int64_t x_sh, int64_t x_st,
                      const float* lambda, int64_t lambda_sb, float* w, void* stream);

/* Bytes of device workspace kvq_attn_decode and kvq_attn_decode_f16 need for
 * this shape: the split-K partial results of the decode-step attention
 * (the pages give no workspace; it is this library's split of the read
 * across the GPU).  D = 128 or 256, else KVQ_ERR_UNSUPPORTED.  The size
 * covers any split count a call with this seq_len may use; the workspace
 * is caller-owned and may be reused across calls in stream order. */
kvq_status kvq_attn_workspace_size(int32_t D, int64_t B, int64_t Hq, int64_t seq_len,
                                   size_t* bytes);

/* Decode-step attention over the int4 cache (the read path fused with
 * attention; the abstract reports its decode latency against fp16 on
 * Gemma-3 1B, head size 256, and Qwen2.5-1.5B, head size 128): for each batch b
 * and query head h, with kv head g = h / (Hq / Hkv),
 *   out[b,h,:] = sum_t softmax_t(sm_scale q[b,h,:] . k^[b,g,t,:]) v^[b,g,t,:]
 * over t < seq_len, where k^ and v^ are the decoded cache rows
 * (codes/scales [B, Hkv, Tcap, ...] as written by kvq_encode, with lambda_k
 * and lambda_v [Hkv, D] shared across the batch).  q is fp16 [B, Hq, D]
 * dense; out is fp16 or fp32 [B, Hq, D] dense.  Scores are taken in the
 * rotated basis (q . k^ = ((R q) / lambda_k) . (lambda_k R k^)) and the
 * value average is rotated back once per head.  Requires Hq % Hkv == 0,
 * 1 <= seq_len <= Tcap < 2^31, and a workspace of kvq_attn_workspace_size
 * bytes.
 * Built for D = 128 and 256, every rotation, code width and group size of
 * the plan (codes [B, Hkv, Tcap, D*bits/8] 16-byte aligned, scales
 * [B, Hkv, Tcap, D/G] 8-byte aligned, lambda 16-byte aligned); plans at D =
 * 96 or 80 return KVQ_ERR_UNSUPPORTED. */
kvq_status kvq_attn_decode(const kvq_plan* plan, const uint16_t* q,
                           const uint8_t* k_codes, const uint16_t* k_scales, const float* lambda_k,
                           const uint8_t* v_codes, const uint16_t* v_scales, const float* lambda_v,
                           int64_t B, int64_t Hq, int64_t Hkv, int64_t Tcap, int64_t seq_len,
                           float sm_scale, void* out, kvq_dtype out_dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Decode-step attention that allocates nothing and takes no workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Arguments, checks
 * and results are those of kvq_attn_decode without the workspace.  The
 * split-K partial results go to a buffer the library keeps in device memory,
 * 16 MiB on each GPU it runs on (held until the process ends).  A call whose
 * partials need more (about B * Hq * splits * (D + 2) * 4 bytes, splits <=
 * 16 at the decode-step shapes) returns KVQ_ERR_WORKSPACE before anything is
 * enqueued.  Every call on one GPU shares that GPU's buffer: calls that
 * overlap on one GPU (on different streams or threads) race, and the caller
 * must order them. */
kvq_status kvq_attn_decode_noalloc(const kvq_plan* plan, const uint16_t* q,
                                   const uint8_t* k_codes, const uint16_t* k_scales, const float* lambda_k,
                                   const uint8_t* v_codes, const uint16_t* v_scales, const float* lambda_v,
                                   int64_t B, int64_t Hq, int64_t Hkv, int64_t Tcap, int64_t seq_len,
                                   float sm_scale, void* out, kvq_dtype out_dtype, void* stream);

/* The same attention over an unquantized fp16 cache k, v [B, Hkv, Tcap, D]
 * (dense, 16-byte aligned): the fp16 cache the abstract compares the int4
 * cache with.  Takes the head size D (128 or 256) instead of a plan, since
 * no quantizer is involved; a row of the cache (Tcap * 2D bytes) must not
 * pass 4 GiB; otherwise as kvq_attn_decode. */
kvq_status kvq_attn_decode_f16(int32_t D, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                               int64_t B, int64_t Hq, int64_t Hkv, int64_t Tcap, int64_t seq_len,
                               float sm_scale, void* out, kvq_dtype out_dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/* ---- Measurement aids (not part of the quantizer; the pages define no
 * such call) ---- */

/* Shader clock probe, for reading benchmark timings: enqueues on `stream`
 * one wave that spins on a dependent chain of `iters` fp32 FMAs (1 to 2^24;
 * 200 take about 4 us at 2.4 GHz) and writes to `out` (device memory, at
 * least 3 uint64, 8-byte aligned, caller-owned) out[0] = shader-clock ticks
 * and out[1] = wall-clock ticks over the chain (out[2] is overwritten too).
 * out[0] / out[1] times the wall-clock rate (kvq_diag_wall_clock_khz) is
 * the shader clock the GPU ran at right after the work queued before it.
 * Errors: KVQ_ERR_INVALID (NULL out, iters out of range), KVQ_ERR_ALIGN,
 * KVQ_ERR_HIP (launch). */
kvq_status kvq_diag_shader_clock(uint64_t* out, int32_t iters, void* stream);

/* Rate of the wall clock the probe reads, in kHz, on the current device. */
kvq_status kvq_diag_wall_clock_khz(int32_t* khz);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
