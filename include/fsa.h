/*
 * fsa.h -- C ABI of the MI355X (gfx950) fused-softmax MX attention library.
 *
 * The operation is the forward pass of Fused-Softmax Attention: FlashAttention-
 * style attention whose Q K^T and P V products run on MX-quantised operands
 * (MXFP8 E4M3, MXFP6 E2M3, MXFP4 E2M1: 32-element blocks sharing one E8M0
 * scale), with the row max frozen speculatively, the exponential approximated
 * and folded together with the MX quantisation of P into the products, the
 * probabilities summed on the matrix cores, and a fallback for rows whose
 * scores exceed the frozen max ("Fused-Softmax for efficient quantized
 * attention", summary; "Moving softmax to matrix operations speeds up AI
 * inference by over 2x", "Read it as" and the "How it works" figure).  The
 * pages give the method only in outline; the exact definitions the kernels
 * implement (frozen-max rule, code map, fallback) are the ones written out
 * step by step in the oracle's module documentation.
 *
 * Conventions for every entry point
 *   - Tensor pointers are DEVICE pointers (HIP device memory, e.g. torch
 *     tensors on a ROCm device).  The caller owns them; the library never
 *     frees caller memory.  Outputs must not alias inputs.
 *   - bf16 tensors are row-major and contiguous.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.  Calls only enqueue work (no host synchronisation); inputs must
 *     stay alive until the stream has run the work.  Device faults surface at
 *     the caller's next synchronisation, not from the call.
 *   - Return value: FSA_OK (0) or a negative fsa_status.  Argument errors are
 *     detected before anything is enqueued.  No C++ exception crosses the ABI.
 *   - Calls are thread-safe.  The library keeps a per-device workspace
 *     (quantised operands) that it allocates on first use and grows as
 *     needed, stream-ordered (hipMallocAsync on the call's stream, the old
 *     buffer freed with hipFreeAsync on the stream of the call that last used
 *     it).  Calls that share a device use the same workspace, so give the
 *     attention calls of one device one stream, or order their streams
 *     yourself.  Calls from several host threads on one stream are
 *     serialised: each call enqueues all of its kernels before the next call
 *     enqueues any.
 */
#ifndef FSA_H
#define FSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fsa_status {
  FSA_OK = 0,
  FSA_ERR_INVALID_ARG = -1,  /* null pointer, non-positive or overflowing size, bad enum */
  FSA_ERR_UNSUPPORTED = -2,  /* valid but not implemented (e.g. head dim other than 64/128) */
  FSA_ERR_HIP = -3,          /* a HIP runtime call or kernel launch failed */
  FSA_ERR_NO_MEMORY = -4,    /* workspace allocation failed */
  FSA_ERR_TOO_LARGE = -5     /* one head exceeds the fixed scratch of fsa_attention_fwd_noalloc */
} fsa_status;

typedef enum fsa_fmt {
  FSA_MXFP8_E4M3 = 0,
  FSA_MXFP6_E2M3 = 1,
  FSA_MXFP4_E2M1 = 2
} fsa_fmt;

/*
 * fsa_quantize_mx -- MX block quantisation of a bf16 tensor.
 *
 * MX operands of the attention products (Fused-Softmax for efficient
 * quantized attention, summary: the pages' kernels take MX operands in three
 * element widths, 8, 6 and 4 bits); encodings
 * and block-scale rule of the OCP Microscaling Formats v1.0 specification:
 * scale X = clamp(floor(log2(amax)) - emax, -127, 127) (X = -127 for an
 * all-zero block), elements x / 2^X rounded to nearest-even and saturated to
 * the largest finite magnitude, the input's sign kept on zeros; a block that
 * holds NaN or Inf gets scale byte 0xFF and zero codes.
 *
 * x_bf16 : device, bf16 [batch][rows][cols].
 * block_along_rows == 0 : blocks are 32 consecutive elements along `cols`.
 *     codes  : device, [batch][rows][ceil(cols/32)*32 * bits/8] bytes.
 *     scales : device, [batch][rows][ceil(cols/32)] E8M0 bytes.
 * block_along_rows == 1 : blocks run along `rows`; the output is transposed.
 *     codes  : device, [batch][cols][ceil(rows/32)*32 * bits/8] bytes.
 *     scales : device, [batch][cols][ceil(rows/32)] E8M0 bytes.
 * Packing (bits = 8, 6, 4): FP8 one byte per element; FP6 a little-endian
 * bit stream with element i of a block at bits [6i, 6i+6) (24 bytes per
 * block); FP4 two elements per byte, the lower-indexed in the low nibble.
 * Padding elements of a partial tail block have code 0.
 * Errors: FSA_ERR_INVALID_ARG for null pointers, sizes <= 0, more than 2^31
 * blocks, an unknown fmt or block_along_rows not 0/1; FSA_ERR_HIP if the
 * launch fails.
 */
int fsa_quantize_mx(const void* x_bf16, void* codes, void* scales_e8m0,
                    int64_t batch, int64_t rows, int64_t cols,
                    int fmt, int block_along_rows, void* stream);

/*
 * fsa_attention_fwd -- fused-softmax attention forward with MX operands.
 *
 * q, k, v : device, bf16 [B][H][S][D]; out : device, bf16 [B][H][S][D];
 *     all four 16-byte aligned (else FSA_ERR_INVALID_ARG).
 * Softmax scale 1/sqrt(D).  D must be 64 or 128 (else FSA_ERR_UNSUPPORTED).
 * fmt : element format of Q, K, V and P (fsa_fmt).  causal : 0 or 1 (key j
 * visible to query i iff j <= i).
 * The call MX-quantises K (blocks along D) and V (blocks along the keys)
 * into the library workspace, then runs one fused kernel that MX-quantises
 * Q times log2(e)/sqrt(D) in its prologue: frozen max from the first 128
 * keys, a score product whose fp32
 * output already is the bit-pattern exponential's exponent field (softmax
 * scale in Q, 2^23 in Q's block scale, max subtraction in the accumulator
 * start), MX quantisation of P in the accumulator epilogue (block shifts
 * applied through the conversion scale), P V and the row sums (P times a
 * ones block) on the matrix cores, and the whole-binade fallback for rows whose
 * scores exceed the frozen max, applied as an exact power-of-two rescale.
 * Errors: FSA_ERR_INVALID_ARG (null pointers, non-positive sizes, B*H*S*D
 * beyond 2^40, unknown fmt, causal not 0/1), FSA_ERR_UNSUPPORTED (D not
 * 64/128, or one head's bf16 rows, S rounded up to 128 times 2*D bytes,
 * reaching 2^31: the kernels address a head with 32-bit buffer offsets),
 * FSA_ERR_NO_MEMORY (workspace), FSA_ERR_HIP (launch).
 */
int fsa_attention_fwd(const void* q, const void* k, const void* v, void* out,
                      int B, int H, int S, int D, int fmt, int causal, void* stream);

/*
 * fsa_attention_bf16_ref -- plain BF16 flash attention (in-house baseline).
 *
 * The unquantised attention the pages measure their speedups against
 * (Fused-Softmax for efficient quantized attention, summary; the vector-unit
 * softmax path of the "How it works" figure): bf16 matrix-core products with fp32 accumulation,
 * exact exponential, online row max and rescaling on the vector units.
 * V is first transposed into the library workspace (B*H*D*S' bf16, S'
 * being S rounded up to 64), which it shares with fsa_attention_fwd.
 * Same tensor layout and errors as fsa_attention_fwd (no fmt).
 */
int fsa_attention_bf16_ref(const void* q, const void* k, const void* v, void* out,
                           int B, int H, int S, int D, int causal, void* stream);

/* Variants of the quantised probabilities P~ (fsa_options.p_variant).  The
 * pages leave the exponential's approximation and the MX quantisation of P
 * open ("Moving softmax to matrix operations speeds up AI inference by over
 * 2x", "Read it as" and the "How it works" figure); the exact definitions
 * are the oracle's.
 *   FSA_P_BLOCK      bit-pattern exponential, each 32-key block of P~ shifted
 *                    to its own E8M0 scale (the default);
 *   FSA_P_ROW_SCALE  one scale for the whole row (every head E4M3); a value
 *                    past 448 sends its row to the fallback pass;
 *   FSA_P_E4M3       E4M3 P~ over FP6/FP4 Q, K, V (every head E2M3 or
 *                    E2M1), through the mixed-width scaled product;
 *   FSA_P_AFFINE     E2M1 codes from one affine rule of the score in the
 *                    code domain, with an exponent-only block scale from the
 *                    block's maximum ("EFQ-Softmax: Exp-Free Quantization
 *                    for Softmax", abstract; every head E2M1);
 *   FSA_P_EXACT_EXP  the vector unit's exp2 in place of the bit pattern:
 *                    P~ is 2^x itself rounded onto the element grid (the
 *                    rounding thresholds of the exact map);
 *   FSA_P_E3M2       E3M2 P~ (FP6 with three exponent bits: eight binades
 *                    below a block's top instead of five, two mantissa bits
 *                    instead of three) over E2M3 Q, K, V (every head E2M3).
 * A variant whose format condition fails gives FSA_ERR_UNSUPPORTED. */
typedef enum fsa_p_variant {
  FSA_P_BLOCK = 0,
  FSA_P_ROW_SCALE = 1,
  FSA_P_E4M3 = 2,
  FSA_P_AFFINE = 3,
  FSA_P_EXACT_EXP = 4,
  FSA_P_E3M2 = 5
} fsa_p_variant;

/* Element strides of strided views: for each tensor, the strides of the
 * batch, head and row indices (element (b, h, s, d) at b*st[0] + h*st[1] +
 * s*st[2] + d).  D is contiguous; each stride a multiple of 8 (16-byte
 * aligned rows) and the row stride at least D.  A [B][S][H][D] tensor viewed
 * as [B][H][S][D], for instance, has strides {S*H*D, D, H*D}. */
typedef struct fsa_layout {
  int64_t q[3], k[3], v[3], out[3];
} fsa_layout;

/* Options of fsa_attention_fwd_ex / fsa_attention_fwd_noalloc.
 * Zero-initialise. */
typedef struct fsa_options {
  /* Added to every frozen max, in binades of the probability (units of
   * log2(e) * q.k / sqrt(D)).  A negative value of a few binades makes every
   * row fall back, a positive one of more than 127 - pl (pl: the placement
   * exponent of P~'s format) re-bases every row downwards; 0 in normal use.
   * Finite with |guess_bias| <= 1024, else FSA_ERR_INVALID_ARG (the fp32
   * score sums taken from the biased reference stay fine enough to measure
   * each row's offset exactly up to that bound). */
  float guess_bias;
  /* Optional device int32 [B][H][S]: receives each row's fallback offset in
   * binades (0 for rows whose scores stayed under the frozen max).  Give
   * both row arrays or neither (else FSA_ERR_INVALID_ARG). */
  int32_t* row_kappa;
  /* Optional device float [B][H][S]: receives each row's frozen max, in
   * the same binade units as guess_bias. */
  float* row_max_guess;
  /* Optional hipEvent_t (as void*) recorded on `stream` between the
   * quantisation kernels and the attention kernel, for kernel-only timing. */
  void* event_after_quantize;
  /* Optional host array of H fsa_fmt values: per-head element format (the
   * hybrid MXFP6/MXFP4 schedule of Fused-Softmax for efficient quantized
   * attention, summary).  Every format runs in the same launches: one
   * quantiser launch for K, one for V and one attention launch pair per
   * call (per 256 heads).  NULL: every head uses `fmt`. */
  const int* head_fmt;
  /* Optional strides of q, k, v and out (strided views); NULL: contiguous
   * [B][H][S][D].  Bad strides give FSA_ERR_INVALID_ARG. */
  const fsa_layout* layout;
  /* fsa_p_variant of P~ (0: the default). */
  int p_variant;
  /* 1: do not launch the fallback pass (a benchmark hook: rows whose scores
   * exceed their frozen max by more than 64 binades then come out wrong,
   * and row_kappa shows them as 65 or more). */
  int skip_fallback_pass;
} fsa_options;

/* fsa_attention_fwd with hooks; opt may be NULL.  Same errors. */
int fsa_attention_fwd_ex(const void* q, const void* k, const void* v, void* out,
                         int B, int H, int S, int D, int fmt, int causal,
                         const fsa_options* opt, void* stream);

/*
 * fsa_debug_operands -- the MX operands exactly as fsa_attention_fwd's
 * kernels consume them (a debug view for bit-exact checks of the operand
 * quantisation; MX operands: Fused-Softmax for efficient quantized attention,
 * summary; block rule as for fsa_quantize_mx).
 *
 * q, k, v : device, bf16 [B][H][S][D], 16-byte aligned; D 64 or 128; every
 *     head takes element format fmt.  Let bits = 8, 6, 4 and
 *     Sk = S rounded up to 128.  Each output pair may be NULL to skip it;
 *     outputs are device memory owned by the caller, code buffers 16-byte
 *     aligned.
 * q_codes  [B][H][S][D*bits/8], q_scales [B][H][S][D/32]: Q times
 *     fp32(log2(e)/sqrt(D)) MX-quantised along D by the attention kernel's
 *     own prologue code, in the packing of fsa_quantize_mx.  Each scale byte
 *     is the block's E8M0 byte raised by 23 (the kernel puts 2^23 on Q's
 *     scale), at most 254; 255 marks a NaN/Inf block.
 * k_codes  [B][H][Sk][D*bits/8]: K quantised along D (padding rows 0);
 * k_scales [B][H][Sk/128][128*D/32]: per 128-key tile, the key-tile order
 *     of the score product (byte of key row r, D block b at
 *     (32 (b%2) + rho) * D/16 + u * D/32 + beta * D/64 + b/2, with r = 64 u
 *     + kk, rho = 8 j + 4 x + kk%4 and (x, beta) = (kk/16%2, kk/32) for FP8,
 *     (kk/32, kk/16%2) otherwise, j = kk/4%4); padding rows 0;
 * v_codes  [B][H][D][Sk*bits/8]: V quantised along the keys, transposed
 *     (padding keys 0);
 * v_scales [B][H][Sk/128][4*D]: per 128-key tile, the byte of row d and
 *     key block kb (0..3) at (32 (kb%2) + d%32) * D/16 + (kb/2) * D/32 + d/32;
 *     padding blocks 0.
 * Errors: FSA_ERR_INVALID_ARG (null inputs, an output pair half NULL,
 * sizes, fmt, alignment), FSA_ERR_UNSUPPORTED (D), FSA_ERR_HIP (launch).
 * Stream-ordered like the other calls.
 */
int fsa_debug_operands(const void* q, const void* k, const void* v, int B, int H, int S, int D,
                       int fmt, void* q_codes, void* q_scales, void* k_codes, void* k_scales,
                       void* v_codes, void* v_scales, void* stream);

/*
 * fsa_attention_fwd_noalloc -- fsa_attention_fwd_ex that allocates nothing.
 *
 * For callers that cannot allocate device memory: code under stream/graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, options, results and errors as fsa_attention_fwd_ex; the
 * quantised operands, per-row offsets and fallback flag live in a fixed
 * 64 MiB device array of the library (one per device, held until the
 * process ends; its address is looked up once per device on the first call
 * there) instead of the growing workspace.  Heads are processed in groups
 * of one batch entry that fit the array, each quantised and attended in
 * turn on `stream`.  FSA_ERR_TOO_LARGE if a single head does not fit (about
 * 264 * S bytes per head at FP8, D = 128; S up to ~250k).  Every call on a
 * device shares that device's array: calls whose kernels overlap in time on
 * one device (different streams) race and must be ordered by the caller;
 * calls from several host threads on one stream are serialised like the
 * other entry points'.  event_after_quantize, if given, is recorded after
 * the first group's quantisation.
 */
int fsa_attention_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                              int B, int H, int S, int D, int fmt, int causal,
                              const fsa_options* opt, void* stream);

/* Static description of a status code (never NULL). */
const char* fsa_strerror(int status);

/* Frees the current device's workspace after the work of the last call
 * that used it (waits for that call's stream).  Returns FSA_OK or
 * FSA_ERR_HIP. */
int fsa_release_workspace(void);

#ifdef __cplusplus
}
#endif

#endif /* FSA_H */
