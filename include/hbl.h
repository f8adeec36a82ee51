/*
 * hbl.h -- C ABI of the H-BitLinear forward (BitNet v2) on AMD Instinct
 * MI355X (gfx950).
 *
 * The method (architecture write-up of "BitNet v2: Native 4-bit Activations
 * with Hadamard Transformation for 1-bit LLMs", §3.4):
 *   - weights are ternarised per tensor with the absmean quantiser
 *     (§3.4 "Weight Quantization", Eq. 1-2);
 *   - each token row of the layer input is rotated by the normalised
 *     Sylvester-Hadamard matrix of its length n = 2^k
 *     (§3.4 "The Hadamard Transformation", Eq. 3-6);
 *   - the rotated row is quantised per token, INT8 absmax (Eq. 7) or INT4
 *     absmean (Eq. 8);
 *   - the layer output is Y = Q_w(W) . Q(X_r)  (§3.4 "H-BitLinear", Eq. 9),
 *     evaluated as an integer matmul of the codes followed by one rescale.
 *
 * Orientation.  Tokens are rows: X is [M][K] row-major, W is [N][K]
 * row-major (out-features by in-features), Y = Xq . Wq^T is [M][N].
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a device pointer unless stated otherwise.
 *     The caller owns every buffer; the library never allocates, frees or
 *     synchronises.  Work is enqueued on `stream` (a hipStream_t; NULL means
 *     the default stream) and the call returns at once.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call enqueues nothing and returns an HBL_ERR_* code.
 *     HBL_ERR_HIP reports a failed launch (detail in hbl_last_error()).
 *     Faults inside a kernel surface at the caller's next synchronisation,
 *     as with any HIP kernel.
 *   - Device pointers must be 16-byte aligned.  Inputs are never written.
 *   - Results are bitwise deterministic (no floating-point atomics).
 *   - M == 0 is a valid no-op.
 *
 * Packed layouts (bit-exact contract):
 *   ternary weights: uint32 [N][K/16].  Word w of row n holds k = 16w..16w+15;
 *       weight j = 4s + b (s, b in 0..3) of the word sits in bits
 *       [8b + 2s, 8b + 2s + 2) as c = q + 1 in {0, 1, 2} (3 is never written).
 *   INT4 codes: uint32 [M][K/8].  Word w of row m holds k = 8w..8w+7;
 *       code j = 4h + b (h in 0..1, b in 0..3) sits in bits [8b + 4h, +4) as a
 *       two's-complement nibble.
 *   INT8 codes: int8 [M][K], natural order.
 *   scales: float [M], the per-token dequantisation factor gamma/127 (INT8)
 *       or beta/sqrt(7) (INT4).
 *   alpha: one float in device memory, the weight scale mean|W|.
 */
#ifndef HBL_H
#define HBL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define HBL_OK 0
#define HBL_ERR_NULL 1      /* a required pointer is NULL */
#define HBL_ERR_SHAPE 2     /* a size or leading dimension is out of range */
#define HBL_ERR_ALIGN 3     /* a pointer or leading dimension is misaligned */
#define HBL_ERR_MODE 4      /* unknown dtype, bits or flag value */
#define HBL_ERR_WORKSPACE 5 /* workspace missing or too small */
#define HBL_ERR_HIP 6       /* a HIP runtime call failed */

/* element types of floating-point inputs */
#define HBL_DTYPE_F32 0
#define HBL_DTYPE_BF16 1

/* flags of hbl_hadamard_quant / hbl_forward (and their _norm_ forms) */
#define HBL_HADAMARD 1 /* rotate each row before quantising (H-BitLinear);
                          without it the row is quantised as is (BitLinear) */

/* output types of hbl_ternary_gemm */
#define HBL_OUT_BF16 0
#define HBL_OUT_F32 1
#define HBL_OUT_I32 2

/* The epsilon of Eq. 1, 7 and 8.  The pages give it no value; 1e-5 is this
 * library's reading, used for weights and activations alike. */
#define HBL_EPS 1e-5f

/* Largest row length accepted with HBL_HADAMARD (the FF width of the pages'
 * 7B model, Table 8). */
#define HBL_MAX_K 16384

/* Largest K of the matmul entry points (hbl_ternary_gemm, hbl_forward and
 * their FP6 x FP4 forms): 2^21.  Up to it every partial sum of the FP6 x
 * FP4 matmul is an integer of magnitude <= 8 K <= 2^24, exact in its fp32
 * accumulators; the int8 path's int32 sums (|sum| <= 256 K) and the 32-bit
 * byte offsets of its 256-row tiles stay in range as well. */
#define HBL_MAX_GEMM_K 2097152

/* Largest output row stride (elements) of the matmul entry points: 2^27.
 * The tile kernels address the rows of one store (up to 8 rows) with
 * 32-bit byte offsets. */
#define HBL_MAX_LDO 134217728

/* Library version, major*10000 + minor*100 + patch. */
int hbl_version(void);

/* Static English text for a status code. */
const char* hbl_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* hbl_last_error(void);

/* Number of compute units of the current device (0 if unknown). */
int hbl_device_cu_count(void);

/* ---------------------------------------------------------------------
 * hbl_ternarize_weights -- absmean ternary weight quantiser
 * (§3.4 "Weight Quantization", Eq. 1-2).
 *
 *   alpha = mean over all N*K entries of |W|   (one scalar per matrix)
 *   q     = RoundClip(W / (alpha + eps), -1, 1), RoundClip(x, a, b) =
 *           min(max(round(x), a), b), round = nearest, ties to even.
 *
 * w:        [N][K] row-major, element type w_dtype (HBL_DTYPE_F32/BF16).
 * w_packed: out, uint32 [N][K/16] in the ternary layout above.
 * alpha:    out, one float (device).
 * ws:       device workspace of at least hbl_ternarize_workspace_size(N, K)
 *           bytes (holds fp64 partial sums); contents are scratch.
 * Shapes:   N >= 1, K >= 16, K % 16 == 0.
 * The |W| sum is accumulated in fp64 in a fixed order (deterministic).
 * ------------------------------------------------------------------- */
size_t hbl_ternarize_workspace_size(int64_t N, int64_t K);
int hbl_ternarize_weights(const void* w, int w_dtype, int64_t N, int64_t K,
                          uint32_t* w_packed, float* alpha, void* ws,
                          size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * hbl_hadamard_f32 -- the per-token rotation alone
 * (§3.4 "The Hadamard Transformation", Eq. 3-6): y[m] = H_k x[m], with
 * H_0 = (1), H_k = 2^{-1/2} [[H_{k-1}, H_{k-1}], [H_{k-1}, -H_{k-1}]]
 * (natural Sylvester order), evaluated as k radix-2 butterfly stages in
 * fp32 followed by one multiplication by 2^{-k/2}.
 *
 * x: [M][ldx] (first K columns used), x_dtype F32 or BF16.
 * y: out, float [M][K] row-major.
 * Shapes: K a power of two, 16 <= K <= HBL_MAX_K; ldx >= K and ldx times the
 * element size a multiple of 16 bytes.
 * ------------------------------------------------------------------- */
int hbl_hadamard_f32(const void* x, int x_dtype, int64_t M, int64_t K,
                     int64_t ldx, float* y, void* stream);

/* ---------------------------------------------------------------------
 * hbl_hadamard_backward_f32 -- backward of the rotation
 * (§3.4 "Gradient Handling Through the Hadamard Transformation", Eq. 10):
 * given dy = dL/d(H x) per token row, writes dx = dL/dx = H^T dy.  H is
 * symmetric and orthogonal, so this is the forward transform applied to dy:
 * the same kernel, the same arithmetic and the same arguments as
 * hbl_hadamard_f32 (dy in place of x, dx in place of y).
 * ------------------------------------------------------------------- */
int hbl_hadamard_backward_f32(const void* dy, int dy_dtype, int64_t M, int64_t K,
                              int64_t lddy, float* dx, void* stream);

/* ---------------------------------------------------------------------
 * hbl_hadamard_quant -- rotation fused with per-token quantisation
 * (Eq. 3-6 followed by Eq. 7 or Eq. 8).
 *
 * With flags & HBL_HADAMARD each row is rotated first (x_r = H x); without
 * it the row is quantised as is (the input of a plain BitLinear).
 *   bits == 8: gamma = max_j |x_r|;  q = RoundClip(127/(gamma+eps) x_r,
 *              -128, 127);  scale = gamma/127.
 *   bits == 4: beta = mean_j |x_r|;  q = RoundClip(sqrt(7)/(beta+eps) x_r,
 *              -8, 7);      scale = beta/sqrt(7).
 * The factor Qmax/(stat+eps) is formed once per row in fp32 with an IEEE
 * divide, and each code is the round-to-nearest-even of x_r * factor,
 * clipped.  How that product is rounded:
 *   - K < 1024 (and every row without HBL_HADAMARD below 1024): the fp32
 *     product fl(x_r * factor) is formed, then rounded to an integer (rint);
 *   - K >= 1024: one fused multiply-add rounds the exact product
 *     v * fl(c * factor) to an integer, v being the un-normalised transform
 *     of the row (fp32) and c = 2^(-k/2) the normalisation (c = 1 without
 *     HBL_HADAMARD; for odd k, c = fl(1/sqrt(K))).  For even k this is the
 *     exact real product x_r * factor rounded once.
 * The two forms give the same code except where x_r * factor lies within
 * half an fp32 ulp of a half-integer (then fl() may land on the half).
 * The statistic: gamma is the exact maximum; beta is a fixed-order fp32
 * tree sum of |x_r| divided by K (the transform's scale applied to the sum).
 *
 * codes:  out, int8 [M][K] (bits 8) or uint32 [M][K/8] (bits 4).
 * scales: out, float [M].
 * rowsum: out, int32 [M], sum of the row's codes (needed by
 *         hbl_ternary_gemm); may be NULL.
 * Shapes: with HBL_HADAMARD K is a power of two, 16 <= K <= HBL_MAX_K;
 *         without it K % 64 == 0 and K <= HBL_MAX_K.  ldx as above.
 * ------------------------------------------------------------------- */
int hbl_hadamard_quant(const void* x, int x_dtype, int64_t M, int64_t K,
                       int64_t ldx, int flags, int bits, void* codes,
                       float* scales, int32_t* rowsum, void* stream);

/* ---------------------------------------------------------------------
 * hbl_norm_hadamard_quant -- hbl_hadamard_quant preceded by the layer's
 * normalisation (§3.4 "H-BitLinear: The Composite Layer", Eq. 9:
 * X_r = Hadamard(LN(X)), LN being RMSNorm).  The pages name RMSNorm without
 * a formula; this library reads it as the usual one:
 *   RMSNorm(x)_k = x_k * r * gain_k,  r = 1/sqrt(mean_j x_j^2 + eps),
 * in fp32 (the mean of squares as a tree sum, r with an IEEE square root
 * and divide), applied before the rotation.
 * gain: device float [K], 16-byte aligned, or NULL for a gain of one.
 * Other arguments, shapes and outputs as hbl_hadamard_quant; the scales
 * are those of the normalised rows.
 * ------------------------------------------------------------------- */
int hbl_norm_hadamard_quant(const void* x, int x_dtype, int64_t M, int64_t K,
                            int64_t ldx, const float* gain, int flags, int bits,
                            void* codes, float* scales, int32_t* rowsum,
                            void* stream);

/* ---------------------------------------------------------------------
 * hbl_ternary_gemm -- integer matmul of activation codes with packed
 * ternary weights and the rescale of Eq. 9:
 *   acc[m][n] = sum_k q_x[m][k] * q_w[n][k]            (exact, int32)
 *   out[m][n] = (scales[m] * alpha) * acc[m][n]        (fp32, then rounded
 *                                                       to nearest-even bf16)
 * codes/scales/rowsum: as written by hbl_hadamard_quant.  rowsum is
 *     required: the kernels multiply the codes with the stored weight
 *     bytes c = q + 1 and subtract sum_k q_x, which the quantiser produces
 *     as it writes the codes.  (A caller holding codes from elsewhere
 *     passes their row sums.)
 * w_packed, alpha:     as written by hbl_ternarize_weights.
 * out_dtype: HBL_OUT_BF16 or HBL_OUT_F32 write the rescaled value;
 *            HBL_OUT_I32 writes acc itself (for exact checks).
 * out: [M][ldo] of out_dtype; ldo >= N, ldo % 4 == 0, ldo <= HBL_MAX_LDO.
 * Shapes: N >= 16, N % 16 == 0, K >= 64, K % 64 == 0, K <= HBL_MAX_GEMM_K.
 * Token counts M <= 128 take a kernel that streams the weights once (one
 * block per 16 output features, the tokens in groups of 16); larger M take
 * the matrix-core tile kernel.
 * ------------------------------------------------------------------- */
int hbl_ternary_gemm(const void* codes, int bits, const float* scales,
                     const int32_t* rowsum, const uint32_t* w_packed,
                     const float* alpha, int64_t M, int64_t N, int64_t K,
                     int out_dtype, void* out, int64_t ldo, void* stream);

/* ---------------------------------------------------------------------
 * hbl_forward -- the whole layer, Eq. 9 without the normalisation layer:
 *   y = bf16( (scale_m * alpha) * sum_k q_x[m][k] q_w[n][k] ),
 * q_x the codes of hbl_hadamard_quant(x, flags, bits).
 * y: out, bf16 [M][ldy]; ldy >= N, ldy % 4 == 0.
 * ws: device workspace of at least hbl_forward_workspace_size(M, N, K,
 *     bits) bytes; it receives the codes, scales and row sums (scratch)
 *     and, when the matmul's 256-token tiles would leave most compute
 *     units idle (fewer than 256 of them, M K >= 2^20, M > 16, K % 512 ==
 *     0), the int32 partial sums of a split of K (at most 32 MiB); integer
 *     sums make the output the same bits with or without the split.
 * Shapes: the union of the rules of hbl_hadamard_quant and
 * hbl_ternary_gemm.  Two kernels are enqueued, except for a few bf16
 * tokens, K a power of two in [1024, 16384]: with HBL_HADAMARD (bits 8 or
 * 4) M <= 4 up to K = 2048, M <= 2 at 4096 and 8192 and M = 1 at 16384;
 * without it (bits 8) M <= 4 up to K = 4096, M <= 2 at 8192 and M = 1 at
 * 16384.  Then one kernel, in
 * which every block rotates (if asked) and quantises the tokens itself
 * while its weights stream in; the codes stay on chip and ws is validated
 * but not written; y is bit-identical to the two-kernel result.
 * ------------------------------------------------------------------- */
size_t hbl_forward_workspace_size(int64_t M, int64_t N, int64_t K, int bits);
int hbl_forward(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                int64_t N, int flags, int bits, const uint32_t* w_packed,
                const float* alpha, void* y, int64_t ldy, void* ws,
                size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * hbl_forward_noalloc -- hbl_forward for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same computation, arguments and result
 * as hbl_forward, without the workspace: the library's own static device
 * array of HBL_NOALLOC_WORKSPACE_BYTES (64 MiB) serves as the workspace.
 * Each GPU the library runs on holds its own copy of that array until the
 * process ends; its device address is looked up on the first call made with
 * the device current (hipGetSymbolAddress; no allocation, no
 * synchronisation).  The call itself allocates nothing.
 * Limit: hbl_forward_workspace_size(M, N, K, bits) <= 64 MiB, else
 * HBL_ERR_WORKSPACE (e.g. M = 2048 at K = 16384 in INT8 needs more).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or threads) race and must be serialised by the
 * caller.  Calls on one stream are ordered and safe.  Nothing in the array
 * needs to start at zero: every byte a call reads was written by the same
 * call.
 * ------------------------------------------------------------------- */
#define HBL_NOALLOC_WORKSPACE_BYTES (64 * 1024 * 1024)
int hbl_forward_noalloc(const void* x, int x_dtype, int64_t M, int64_t K,
                        int64_t ldx, int64_t N, int flags, int bits,
                        const uint32_t* w_packed, const float* alpha, void* y,
                        int64_t ldy, void* stream);

/* ---------------------------------------------------------------------
 * hbl_norm_forward -- the whole layer of Eq. 9 with its normalisation:
 * hbl_norm_hadamard_quant(x, gain, flags, bits) then hbl_ternary_gemm.
 * Arguments as hbl_forward plus gain (as hbl_norm_hadamard_quant); the
 * workspace is hbl_forward_workspace_size(M, N, K, bits) bytes.
 * ------------------------------------------------------------------- */
int hbl_norm_forward(const void* x, int x_dtype, int64_t M, int64_t K,
                     int64_t ldx, const float* gain, int64_t N, int flags,
                     int bits, const uint32_t* w_packed, const float* alpha,
                     void* y, int64_t ldy, void* ws, size_t ws_bytes,
                     void* stream);

/* ---------------------------------------------------------------------
 * hbl_ternarize_weights_rotated -- the weight side of the "weight and
 * activation rotation" variant (§3.4 "Ablation Study: Why Activation-Only
 * Hadamard Transformation", Table 5): the matrix quantised is W H^T instead
 * of W, so that Q_w(W H^T) . Q(H x) approximates W x.  Row n of W H^T is
 * the rotation of row n of W (H is symmetric): each row goes through the
 * transform of hbl_hadamard_f32 (fp32) and the fp32 result through the
 * quantiser of hbl_ternarize_weights.  Pair it with HBL_HADAMARD on the
 * activations.
 * w, w_packed, alpha: as hbl_ternarize_weights.
 * ws: device workspace of at least hbl_ternarize_rotated_workspace_size(N,
 *     K) bytes (the rotated fp32 matrix, then the partial sums); scratch.
 * Shapes: N >= 1; K a power of two, 16 <= K <= HBL_MAX_K.
 * ------------------------------------------------------------------- */
size_t hbl_ternarize_rotated_workspace_size(int64_t N, int64_t K);
int hbl_ternarize_weights_rotated(const void* w, int w_dtype, int64_t N, int64_t K,
                                  uint32_t* w_packed, float* alpha, void* ws,
                                  size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------
 * hbl_kv_quant -- post-RoPE QKV / KV-cache quantiser (§3.4 "QKV Attention
 * Quantization: Post-RoPE INT4/3-bit"): every head of every token is
 * quantised to unsigned b-bit integers with the absmax function, without
 * calibration; the KV heads of the [BOS] token are kept at 8 bits.
 * The pages give no formula for the unsigned mapping; this library reads it
 * as Eq. 7's absmax quantiser at b bits shifted into [0, 2^b - 1]:
 *   gamma = max |x| over the head's D elements, Q = 2^(b-1) - 1,
 *   u = RoundClip(x * Q / (gamma + eps), -2^(b-1), 2^(b-1) - 1) + 2^(b-1),
 *   scale = gamma / Q,  so that x ~ (u - 2^(b-1)) * scale.
 * x: [B][S][H][D] contiguous (B sequences of S positions, H heads of D
 *    elements), x_dtype F32 or BF16, 16-byte aligned.
 * bits: 3, 4 or 8.
 * codes: out, [B][S][H][D * bits / 8] bytes: bits 8 one byte per code;
 *    bits 4 code 2i in the low nibble of byte i; bits 3 eight codes per
 *    three bytes, code j of the eight at bits [3j, 3j + 3) of their 24-bit
 *    little-endian value.  16-byte aligned.
 * scales: out, float [B][S][H].
 * keep_bos8: nonzero -- position 0 of every sequence (the [BOS] token) is
 *    also written at 8 bits to bos_codes [B][H][D] bytes and bos_scales
 *    float [B][H] (its low-bit slot in codes is written as well).
 * Shapes: D a power of two, 32 <= D <= 2048; S, H >= 1; B == 0 is a no-op.
 * ------------------------------------------------------------------- */
int hbl_kv_quant(const void* x, int x_dtype, int64_t B, int64_t S, int64_t H,
                 int64_t D, int bits, int keep_bos8, void* codes, float* scales,
                 void* bos_codes, float* bos_scales, void* stream);

/* =====================================================================
 * INT4 on the FP6 x FP4 matrix cores.
 *
 * INT4 activation codes in [-8, 7] are exact 6-bit floats E3M2 (OCP MX
 * "BF6": sign, 3 exponent bits with bias 3, 2 mantissa bits) and ternary
 * weights exact 4-bit floats E2M1 (sign, 2 exponent bits with bias 1, 1
 * mantissa bit); every product is an integer of magnitude <= 8 and the
 * fp32 accumulator of v_mfma_f32_32x32x64_f8f6f4 holds every partial sum
 * exactly (|sum| <= 8 K < 2^24).  The matmul is therefore the same exact
 * integer matmul as hbl_ternary_gemm (same int32 values, same bf16
 * outputs), at twice the per-clock rate of the int8 matrix cores.  It is
 * the INT4 path of Eq. 8-9 (§3.4) on gfx950's low-precision matrix cores.
 *
 * Operand layouts (bit-exact contract).  Each is stored as the matmul's
 * LDS stage images, so that its stage loads are contiguous copies.
 *   MX6 codes: groups of 32 codes (k = 32 g .. 32 g + 31 of a token row) as
 *       192-bit little-endian fields, code e at bits [6 e, 6 e + 6) as an
 *       E3M2 float (0 = 0b000000, 1 = 0b001100, 2 = 0b010000,
 *       3 = 0b010010, 4 = 0b010100, 5 = 0b010101, 6 = 0b010110,
 *       7 = 0b010111, 8 = 0b011000, bit 5 the sign).  Tile (B, s) of 24576
 *       bytes holds token rows 256 B .. 256 B + 255 and codes
 *       128 s .. 128 s + 127 at byte offset (B * (K / 128) + s) * 24576: for
 *       row r = m % 256 and group gi = g % 4 of the tile, the field's first
 *       16 bytes at 16 * (4 r + (gi ^ ((r >> 2) & 3))), its last 8 bytes at
 *       16384 + 16 * (2 r + ((gi >> 1) ^ ((r >> 3) & 1))) + 8 * (gi & 1).
 *       The buffer holds whole 256-row blocks: hbl_mx_codes_bytes(M, K)
 *       bytes (rows past M are padding, never read into an output).
 *   MX4 weights: uint32 words, two bits per weight: for the word of
 *       k = 16 w .. 16 w + 15 of a feature row and n = 0..7,
 *       bit 4n+1 = (q[16w+n] != 0), bit 4n+3 = (q[16w+n] < 0),
 *       bit 4n = (q[16w+8+n] != 0), bit 4n+2 = (q[16w+8+n] < 0), so that
 *       word & 0xAAAAAAAA and (word << 1) & 0xAAAAAAAA are the E2M1 codes
 *       of the two halves.  Tile (b, s) of 4096 bytes holds feature rows
 *       128 b .. 128 b + 127 and k = 128 s .. 128 s + 127 at byte offset
 *       (b * (K / 128) + s) * 4096: row r's k = 128 s + 64 u .. + 63 (four
 *       words) at 16 * (2 r + (u ^ ((r >> 3) & 1))).  Rows past N are
 *       zero; the buffer holds hbl_mx_weights_bytes(N, K) bytes.
 * ===================================================================== */

/* Buffer sizes of the two layouts. */
size_t hbl_mx_codes_bytes(int64_t M, int64_t K);
size_t hbl_mx_weights_bytes(int64_t N, int64_t K);

/* hbl_prepare_weights_mx -- ternary layout (hbl_ternarize_weights) to the
 * MX4 layout (w_mx: hbl_mx_weights_bytes(N, K) bytes).  Offline, once per
 * matrix.  Shapes: N >= 1, K % 128 == 0. */
int hbl_prepare_weights_mx(const uint32_t* w_packed, int64_t N, int64_t K,
                           uint32_t* w_mx, void* stream);

/* hbl_hadamard_quant_mx -- hbl_hadamard_quant with bits = 4 (Eq. 8, after
 * the rotation with HBL_HADAMARD), codes written in the MX6 layout:
 * codes_mx hbl_mx_codes_bytes(M, K) bytes, scales [M] (beta / sqrt(7)).  The
 * same codes and scales as hbl_hadamard_quant(..., bits = 4).
 * Shapes: K a power of two, 1024 <= K <= HBL_MAX_K; ldx as there. */
int hbl_hadamard_quant_mx(const void* x, int x_dtype, int64_t M, int64_t K,
                          int64_t ldx, int flags, void* codes_mx, float* scales,
                          void* stream);

/* hbl_ternary_gemm_mx -- hbl_ternary_gemm for MX6 codes and MX4 weights:
 *   out[m][n] = (scales[m] * alpha) * sum_k q_x[m][k] q_w[n][k]
 * (HBL_OUT_I32: the exact sum).  No row sums are needed.
 * Shapes: N >= 16, N % 16 == 0; K >= 512, K % 512 == 0, K <= HBL_MAX_GEMM_K;
 * ldo as there. */
int hbl_ternary_gemm_mx(const void* codes_mx, const float* scales,
                        const uint32_t* w_mx, const float* alpha, int64_t M,
                        int64_t N, int64_t K, int out_dtype, void* out,
                        int64_t ldo, void* stream);

/* hbl_forward_mx -- the INT4 layer of Eq. 9 on this path:
 * hbl_hadamard_quant_mx then hbl_ternary_gemm_mx (bf16 output), the same
 * result as hbl_forward(..., bits = 4).  ws: at least
 * hbl_forward_mx_workspace_size(M, N, K) bytes: the MX6 codes, the scales
 * and, when the 256-token tiles alone would leave most compute units idle
 * (fewer than 256 tiles), room for the exact partial sums of a split of K
 * (at most 32 MiB), whose sum is order-independent, so the output is the
 * same bits with or without the split.
 * Shapes: the union of the two calls' rules. */
size_t hbl_forward_mx_workspace_size(int64_t M, int64_t N, int64_t K);
int hbl_forward_mx(const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                   int64_t N, int flags, const uint32_t* w_mx, const float* alpha,
                   void* y, int64_t ldy, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HBL_H */
