/*
 * bitlinear.h - C ABI of libbitlinear.so, the MI355X (gfx950) BitNet b1.58 BitLinear
 * forward.
 *
 * The operation (pages: aratech.ae "BitNet b1.58: Microsoft's 1-bit LLM that runs a
 * 100B model on one CPU", sub-sections "Ternary weights {-1, 0, +1}" and "BitLinear:
 * the building block"; bhfrc.com news 56965, sections 1.1 and 4.1):
 *
 *   1. weights W[N][K] (out x in) -> gamma = mean |W| over the whole tensor, codes
 *      q = clamp(round(W / gamma), -1, 1) in {-1, 0, +1}, packed at 2 bits per weight
 *      with the code table 00 -> 0, 01 -> +1, 10 -> -1, 11 -> padding;
 *   2. activations x[M][K] -> per token (row) a[m] = max_k |x[m][k]|, int8 codes
 *      xq = clamp(round(x * 127 / a), -127, 127);
 *   3. acc[m][n] = sum_k xq[m][k] * q[n][k], exact in int32 (each term adds, subtracts
 *      or skips an activation);
 *   4. y[m][n] = acc[m][n] * gamma * a[m] / 127 in fp32.
 *
 * Numeric conventions fixed by this library (the pages leave them open):
 *   - gamma is the exact mean of |W| rounded to the nearest fp32 (ties to even); it
 *     does not depend on summation order, so it is reproducible bit for bit.
 *   - "round" is round-half-to-even; the ternarise decision is t = fl32(W * fl32(1/gamma)),
 *     the activation decision t = fl32(x * fl32(127/a)); gamma == 0 gives all-zero codes,
 *     a zero row gives zero codes and a[m] = 0.
 *   - The packed layout (below) is designed for gfx950 loads; it is not a file format
 *     from the pages.
 *
 * Packed weight layout.  N_pad = roundup(N, 16), K_pad = roundup(K, 256).  The buffer
 * holds N_pad*K_pad/4 bytes as 1024-byte tiles; tile (nb, c) starts at byte
 * (nb*(K_pad/256) + c)*1024 and covers rows 16nb..16nb+15, columns 256c..256c+255.  In a
 * tile, row r and column offset kk sit in the little-endian 32-bit word at byte
 * 16*(16*(kk/64) + r) + 4*((kk%64)/16), bits 8*(kk%4) + 2*((kk%16)/4) (+1).  So each
 * 16-byte slot is 64 consecutive columns of one row, one 64-lane wave load covers a
 * whole tile, and (word >> 2f) & 0x03030303 yields four consecutive codes, one per byte.
 * Entries outside N x K hold the padding code 11 (decoded as 0).
 *
 * Activation layout.  xq is int8 [M][K_pad], row-major, padding columns zero.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers (HIP global memory) owned by the caller;
 *     the library allocates nothing and keeps no state between calls.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only enqueue work
 *     and return; completion is observed through the stream.
 *   - Arguments are validated on the host before anything is enqueued; errors are
 *     returned synchronously as a negative bl_status and nothing is launched.  A failed
 *     launch returns BL_ERR_HIP.  Device data (NaN/Inf) is never inspected: inputs must
 *     be finite.  An activation row that is not all zero needs a finite fp32 scale
 *     127 / a: a row whose largest magnitude a is below 127 / FLT_MAX (about 3.7e-37)
 *     gets unspecified codes.
 *   - Work enqueued on one stream may run concurrently with work on another; buffers
 *     shared between streams are the caller's responsibility.
 */
#ifndef BITLINEAR_H_
#define BITLINEAR_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BL_OK = 0,
  BL_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad alignment, small workspace */
  BL_ERR_UNSUPPORTED = -2, /* a shape or dtype this build does not handle */
  BL_ERR_HIP = -3          /* a HIP runtime call or kernel launch failed */
} bl_status;

typedef enum { BL_F32 = 0, BL_BF16 = 1 } bl_dtype;

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int bitlinear_version(void);

/* Static text for a bl_status value (never NULL). */
const char* bitlinear_status_string(int status);

/* Host-only size helpers; return -1 for arguments < 1. */
int64_t bitlinear_n_pad(int64_t N);                         /* roundup(N, 16)            */
int64_t bitlinear_k_pad(int64_t K);                         /* roundup(K, 256)           */
int64_t bitlinear_packed_bytes(int64_t N, int64_t K);       /* N_pad * K_pad / 4         */
int64_t bitlinear_wq_workspace_bytes(int64_t N, int64_t K); /* scratch for the quantiser */

/*
 * Step 1 - weight quantiser (aratech.ae, "Ternary weights {-1, 0, +1}"; code table from
 * bhfrc.com section 4.1).
 *   W         [N][K] fp32, row-major, N = out_features, K = in_features. 4-byte aligned.
 *   packed    out: bitlinear_packed_bytes(N, K) bytes in the layout above, 16-byte aligned.
 *   gamma     out: one fp32, the absmean scale (written on the device).
 *   workspace device scratch of at least bitlinear_wq_workspace_bytes(N, K) bytes,
 *             8-byte aligned; it is initialised by the call itself.
 * Requires 1 <= N, K and N*K < 2^40.  Not safe to run concurrently on one workspace.
 */
int bitlinear_quantize_weights(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                               void* workspace, int64_t ws_bytes, void* stream);

/*
 * Step 1 without any allocation, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same result as bitlinear_quantize_weights, with the quantiser's scratch (the exponent
 * bins and 1/gamma, 2304 bytes) in a static device array of the library instead of a
 * caller workspace.  Each GPU holds its own copy until the process ends; it is looked up
 * on the first call on a device (that device current).  The call allocates nothing.
 * Arguments and limits as bitlinear_quantize_weights (N * K < 2^40, else
 * BL_ERR_UNSUPPORTED; the scratch does not grow with the shape).  The scratch is cleared
 * by a kernel at the start of every call; calls that overlap on one GPU (other streams,
 * other host threads) share it and race.
 */
int bitlinear_quantize_weights_noalloc(const float* W, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                                       void* stream);

/*
 * Step 2 - per-token absmax int8 activation quantiser (aratech.ae, "BitLinear: the
 * building block": the largest magnitude of each token maps to 127).
 *   X       [M][K] fp32 (dt = BL_F32) or bf16 (dt = BL_BF16), row-major, element-aligned.
 *   Xq      out: int8 [M][K_pad], 16-byte aligned; columns K..K_pad-1 are set to 0.
 *   absmax  out: fp32 [M], a[m] = max_k |X[m][k]|.
 *   rowsum  out (nullable): int32 [M], sum_k Xq[m][k], exact (|sum| <= 127 K).
 */
int bitlinear_quantize_acts(const void* X, int dt, int64_t M, int64_t K, int8_t* Xq, float* absmax,
                            int32_t* rowsum, void* stream);

/*
 * Steps 3 + 4 - packed-ternary x int8 contraction with exact int32 accumulation
 * (bhfrc.com section 1.1: add / subtract / skip) and the rescale to fp32.
 *   packed  from bitlinear_quantize_weights for the same N, K; 16-byte aligned.
 *   gamma   device pointer to the fp32 weight scale.
 *   Xq      int8 [M][K_pad] and absmax fp32 [M] from bitlinear_quantize_acts.
 *   Y       out (nullable): fp32 [M][N], y = acc * gamma * absmax[m] / 127.
 *   acc     out (nullable): int32 [M][N], the exact accumulators.
 * At least one of Y and acc must be non-null.  M = 1..16 runs the decode kernels
 * (HBM-streaming, MFMA on in-register decoded weights), and so does M = 17..64 in token
 * groups of 16 sharing each decoded weight fragment where that is estimated faster (every
 * row block re-reads the token rows: short rows and few row blocks); other M runs the
 * prefill GEMM
 * (activations staged in LDS, weights decoded in registers, int8 MFMA).  |acc| <= 127*K
 * must fit int32: K <= 2^24.
 */
int bitlinear_forward(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                      int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, void* stream);

/*
 * bitlinear_forward with a caller workspace (steps 3 + 4, as bitlinear_forward; the same
 * arguments and results, bit for bit).  The workspace lets the prefill GEMM even out a
 * partial last round of output tiles: where the tiles need more than one round of the
 * GPU's resident workgroups, the whole rounds run as in bitlinear_forward, and the tiles
 * left over are split along K (the contraction index) into ranges computed by different
 * workgroups, each writing its exact int32 partial tile to the workspace; a second launch
 * on the stream adds the partials (integer addition: the result does not depend on the
 * order) and writes y / acc.  The planner takes the split only where the partial tiles
 * stay within 8 MiB (their bytes are written and read once more, next to the fp32
 * output); otherwise bitlinear_forward_ws_bytes returns 0 and the call is
 * bitlinear_forward (workspace may then be null).
 *   workspace  device memory of at least bitlinear_forward_ws_bytes(M, N, K) bytes,
 *              256-byte aligned, owned by the caller; its contents on entry do not
 *              matter and nothing in it carries over between calls.  Calls that share a
 *              workspace must not overlap (one stream, or events between streams).
 *   ws_bytes   its size in bytes.
 * Errors: those of bitlinear_forward; BL_ERR_INVALID_ARG when the workspace is needed and
 * is null, misaligned or smaller than required (nothing enqueued).
 */
int64_t bitlinear_forward_ws_bytes(int64_t M, int64_t N, int64_t K);
int bitlinear_forward_ws(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                         int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, void* workspace, int64_t ws_bytes,
                         void* stream);
/*
 * Host-only description of the launches bitlinear_forward_ws makes for (M, N, K); no
 * device work.  out[0..5] as bitlinear_forward_plan; where the split tail runs, out[0] = 6,
 * out[1] = workgroups of the first launch, out[2] = threads, out[3] / out[4] = output tile
 * rows / columns, out[5] = 1, out[6] = rounds of whole tiles, out[7] = tiles split along K,
 * out[8] = K ranges per split tile, out[9] = 256-column chunks per range (out[6..9] are 0
 * otherwise).  Returns BL_OK or BL_ERR_INVALID_ARG (as bitlinear_forward_plan).
 */
int bitlinear_forward_ws_plan(int64_t M, int64_t N, int64_t K, int32_t out[10]);

/*
 * Steps 2 + 3 + 4 in one call: per-token activation quantisation, contraction and
 * rescale, for inference on un-quantised activations.
 *   X       [M][K] fp32 (dt = BL_F32) or bf16 (dt = BL_BF16), row-major.
 *   Xq      out: int8 [M][K_pad] codes, 16-byte aligned (as bitlinear_quantize_acts).
 *   absmax  out: fp32 [M] (as bitlinear_quantize_acts).
 *   Y, acc  as bitlinear_forward (at least one non-null).
 * Results are identical to bitlinear_quantize_acts followed by bitlinear_forward.  For a
 * few tokens (M <= 4) with K a multiple of 8 (bf16) or 4 (fp32), a 16-byte aligned X and
 * K up to a size limit that depends on M and dt (at least 8192), one kernel launch does
 * all three steps: each workgroup computes the per-token absmax from the activation
 * pieces its waves hold, and each lane quantises its own pieces.  For 5 to 16 tokens with
 * bf16 X, K a multiple of 8, K <= 7168 and M K <= 65536, one kernel launch does the same with the
 * whole M x K input quantised into LDS by every workgroup (each token row held by one
 * wave, so the row's absmax is a wave reduction).  Otherwise the two kernels run back to back
 * (bitlinear_forward_fused_plan tells which).
 */
int bitlinear_forward_fused(const uint8_t* packed, const float* gamma, const void* X, int dt, int64_t M, int64_t N,
                            int64_t K, float* Y, int32_t* acc, int8_t* Xq, float* absmax, void* stream);

/* One weight matrix of a grouped call: device pointers as in bitlinear_forward. */
typedef struct {
  const uint8_t* packed; /* from bitlinear_quantize_weights for (N, K); 16-byte aligned */
  const float* gamma;    /* its fp32 weight scale                                      */
  int64_t N;             /* its output features                                        */
  float* Y;              /* out (nullable): fp32 [M][N]                                */
  int32_t* acc;          /* out (nullable): int32 [M][N]; Y or acc must be non-null    */
} bl_matrix;

/*
 * Several projections of one input (for instance Q, K and V, or gate and up), each with
 * its own packed weights and scale: the activation quantisation runs once and the
 * contractions of all matrices share its codes.  mats is a HOST array of count
 * descriptors (1 <= count <= 8), all with in_features K; X, dt, M, K, Xq and absmax as
 * bitlinear_forward_fused.  Results are identical to bitlinear_forward_fused on each
 * matrix.  For M <= 4 with a 16-byte aligned X, when bitlinear_forward_fused_plan(M,
 * sum of N_pad, K, dt) reports a fused kernel with activations in registers, the whole
 * group is one kernel launch (workgroups take the row blocks of the matrices in order);
 * likewise for 5..16 tokens under the conditions of the LDS form of
 * bitlinear_forward_fused.  Otherwise the quantiser runs once, then one forward launch for
 * the whole group (5..16 tokens, K up to 4096) or one per matrix.
 */
int bitlinear_forward_grouped(const bl_matrix* mats, int count, const void* X, int dt, int64_t M, int64_t K,
                              int8_t* Xq, float* absmax, void* stream);

/*
 * Sub-layer normalisation in front of step 2.  The aratech.ae article ("BitLinear: the
 * building block") puts a simplified LayerNorm (SubLN) right before the activation
 * quantiser.  This library reads it as RMS normalisation with no centring and no bias:
 *     n[m][k] = X[m][k] * gain[k] / sqrt(mean_k X[m][k]^2 + eps),
 * and quantises n per token as step 2.  Absmax quantisation gives a row and any positive
 * multiple of it the same codes, so the codes are those of h = fl32(X * gain) under
 * step 2's arithmetic (bit for bit), and the scale written out is
 *     scale[m] = max_k |h[m][k]| / sqrt(mean_k X[m][k]^2 + eps)   (= max_k |n[m][k]|),
 * evaluated in fp64 from an fp64 sum of squares and rounded once to fp32; an all-zero h
 * gives zero codes and scale 0.  scale takes the place of absmax in bitlinear_forward.
 *   X      [M][K] fp32 (dt = BL_F32) or bf16 (dt = BL_BF16), row-major.
 *   gain   fp32 [K] per-feature gain (device, 4-byte aligned), or NULL for all ones.
 *   eps    finite, >= 0 (BL_ERR_INVALID_ARG otherwise).
 *   Xq     out: int8 [M][K_pad], 16-byte aligned; scale out: fp32 [M].
 */
int bitlinear_subln_quantize_acts(const void* X, int dt, int64_t M, int64_t K, const float* gain, float eps,
                                  int8_t* Xq, float* scale, void* stream);

/*
 * Sub-layer normalisation + steps 2, 3, 4: bitlinear_forward_fused with the normalising
 * quantiser above in place of step 2 (Xq and scale out as bitlinear_subln_quantize_acts;
 * the rest as bitlinear_forward_fused).  Results are identical to
 * bitlinear_subln_quantize_acts followed by bitlinear_forward.  For M <= 4 with a
 * 16-byte aligned X and gain, K a multiple of 8 (bf16) or 4 (fp32) and K within a size
 * limit that depends on M and dt (bitlinear_forward_subln_plan tells), one kernel launch
 * does all of it; otherwise the two kernels run back to back.
 */
int bitlinear_forward_subln(const uint8_t* packed, const float* gamma, const void* X, int dt, int64_t M, int64_t N,
                            int64_t K, const float* gain, float eps, float* Y, int32_t* acc, int8_t* Xq,
                            float* scale, void* stream);

/*
 * bitlinear_forward_grouped behind the sub-layer normalisation (gain, eps as above): one
 * normalising quantisation shared by all matrices of the group, in one launch under the
 * conditions of bitlinear_forward_subln (with N the sum of N_pad over the group).
 */
int bitlinear_forward_grouped_subln(const bl_matrix* mats, int count, const void* X, int dt, int64_t M, int64_t K,
                                    const float* gain, float eps, int8_t* Xq, float* scale, void* stream);

/*
 * Host-only: what bitlinear_forward_subln does for (M, N, K, dt), in the format of
 * bitlinear_forward_fused_plan (out[0] = 3: one fused launch with activations in
 * registers; otherwise the plan of the forward that follows the normalising quantiser).
 */
int bitlinear_forward_subln_plan(int64_t M, int64_t N, int64_t K, int dt, int32_t out[6]);

/*
 * A gate / up pair of projections of one input with the squared-ReLU gating of the
 * feed-forward layers (aratech.ae, "BitLinear: the building block": squared ReLU in the
 * feed-forward layers), read for the pair as
 *     H[m][n] = relu(y_gate[m][n])^2 * y_up[m][n]        (fp32, relu(v) = max(v, 0)),
 * where y_gate and y_up are the outputs bitlinear_forward would give for the two
 * matrices (both N x K) on the same quantised activations.
 *   X, dt, Xq, scale  as bitlinear_forward_fused (subln = 0) or bitlinear_forward_subln
 *                     (subln = 1, with gain and eps as there; ignored when subln = 0).
 *   H                 out: fp32 [M][N].
 *   workspace         device scratch of at least bitlinear_gated_relu2_workspace_bytes(M, N)
 *                     bytes (4-byte aligned), used only when the pair does not run as one
 *                     kernel (bitlinear_forward_gated_relu2_plan tells); may be NULL when it
 *                     does.  A missing or short workspace then gives BL_ERR_INVALID_ARG.
 * For M <= 4 with a 16-byte aligned X (and gain), under the size limits of
 * bitlinear_forward_fused / bitlinear_forward_subln and runs of at most 8 tiles per wave,
 * one kernel streams the same 16-row block of both matrices per workgroup with one set of
 * activation registers and applies the gating in its epilogue.  Otherwise: the quantiser,
 * the two forwards (gate into H, up into the workspace) and an elementwise gating kernel.
 */
int64_t bitlinear_gated_relu2_workspace_bytes(int64_t M, int64_t N);
int bitlinear_forward_gated_relu2(const uint8_t* gate_packed, const float* gate_gamma, const uint8_t* up_packed,
                                  const float* up_gamma, const void* X, int dt, int64_t M, int64_t N, int64_t K,
                                  int subln, const float* gain, float eps, float* H, int8_t* Xq, float* scale,
                                  void* workspace, int64_t ws_bytes, void* stream);
/* Host-only: out[0] = 3 when the pair runs as one kernel (format of
 * bitlinear_forward_fused_plan), otherwise the plan of each forward. */
int bitlinear_forward_gated_relu2_plan(int64_t M, int64_t N, int64_t K, int dt, int subln, int32_t out[6]);

/*
 * Steps 3 + 4 by table lookups: the lookup-table technique of the CPU kernels the
 * bhfrc.com write-up (section 4) and the aratech.ae article describe, built on gfx950 LDS
 * for comparison with bitlinear_forward.  Same arguments, layouts and results (acc
 * bit-exact, y as bitlinear_forward).  For each pair of activations that share a nibble
 * of the packed layout (columns c and c + 4), a 16-entry int16 table holds the pair's
 * contribution for every nibble value; each packed byte is then two lookups and two adds.
 * Supported for M <= 4 and K with M * roundup(K, 256) within the table budget
 * (bitlinear_forward_lut_plan); otherwise BL_ERR_UNSUPPORTED and nothing is enqueued.
 */
int bitlinear_forward_lut(const uint8_t* packed, const float* gamma, const int8_t* Xq, const float* absmax,
                          int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, void* stream);
/* Host-only: out[0] = 4, out[1] = workgroups, out[2] = threads, out[3] = 1, out[4] = K
 * tiles per wave, out[5] = LDS bytes of tables.  BL_ERR_UNSUPPORTED where the shape does
 * not fit, BL_ERR_INVALID_ARG for invalid sizes. */
int bitlinear_forward_lut_plan(int64_t M, int64_t N, int64_t K, int32_t out[6]);

/*
 * 1-bit sign-binary weights, the contrast point to the ternary path (lpnh.cn news
 * 2861808, section 2.1: binary weights sign(W) with a scaling factor that compensates the
 * lost magnitude).  Readings: q = +1 for W >= 0 (including -0.0), -1 for W < 0; the scale
 * beta is the exact mean |W| (as gamma); activations, contraction and rescale are steps
 * 2-4 with beta in place of gamma.  One bit per weight: half the packed bytes.
 *
 * Binary layout.  N_pad = roundup(N, 16), KB_pad = roundup(K, 512); N_pad * KB_pad / 8
 * bytes of 1024-byte tiles, tile (nb, c) at (nb * (KB_pad / 512) + c) * 1024 covering rows
 * 16 nb .. 16 nb + 15 and columns 512 c .. 512 c + 511.  Row r, column offset kk: with
 * s = kk / 256, g = (kk % 256) / 64, i = (kk % 64) / 16, e = kk % 16, the little-endian
 * 32-bit word at byte 16 * (16 g + r) + 4 * (2 s + i / 2) holds the weight at bit
 * 8 * (e % 4) + 4 * (i % 2) + e / 4: 1 = +1, 0 = -1.  Bits outside N x K are 0.
 *
 * bitlinear_quantize_weights_binary: arguments as bitlinear_quantize_weights (packed:
 *   bitlinear_packed_bytes_binary(N, K) bytes, 16-byte aligned; beta: device fp32).
 * bitlinear_forward_binary: arguments as bitlinear_forward with the binary buffer and
 *   beta; M = 1..4 and K within the plan (bitlinear_forward_binary_plan), otherwise
 *   BL_ERR_UNSUPPORTED and nothing is enqueued.
 */
int64_t bitlinear_kb_pad(int64_t K);                          /* roundup(K, 512)            */
int64_t bitlinear_packed_bytes_binary(int64_t N, int64_t K);  /* N_pad * KB_pad / 8         */
int bitlinear_quantize_weights_binary(const float* W, int64_t N, int64_t K, uint8_t* packed, float* beta,
                                      void* workspace, int64_t ws_bytes, void* stream);
int bitlinear_forward_binary(const uint8_t* packed, const float* beta, const int8_t* Xq, const float* absmax,
                             int64_t M, int64_t N, int64_t K, float* Y, int32_t* acc, void* stream);
/* Host-only: out[0] = 5, out[1] = workgroups, out[2] = threads, out[3] = 1, out[4] = binary
 * tiles per wave, out[5] = 0; BL_ERR_UNSUPPORTED where the shape does not fit. */
int bitlinear_forward_binary_plan(int64_t M, int64_t N, int64_t K, int32_t out[6]);

/*
 * Host-only description of the launch bitlinear_forward would make for (M, N, K); no
 * device work.  out[0] = kernel (1 = decode, 2 = prefill), out[1] = workgroups,
 * out[2] = threads per workgroup, out[3] = decode: 16-row output blocks per workgroup,
 * prefill: output tile rows, out[4] = decode: where the activations live (0 = loaded with
 * each weight tile, 1 = staged in LDS, 2 = held in registers and broadcast across lanes),
 * prefill: output tile columns, out[5] = decode: dynamic LDS bytes (out[4] = 1) or K
 * tiles per wave (out[4] = 2), else 0; prefill: K groups that split each tile's K range
 * (1 or 2; a group is four waves, or eight for the 384-column tiles, which run one group).
 * Returns BL_OK or BL_ERR_INVALID_ARG (same size rules as
 * bitlinear_forward, null out).
 */
int bitlinear_forward_plan(int64_t M, int64_t N, int64_t K, int32_t out[6]);

/*
 * Host-only description of what bitlinear_forward_fused does for (M, N, K) and activation
 * type dt, for a 16-byte aligned X; no device work.  out[0] = 3 when one fused kernel
 * quantises and contracts (out[1..3] as bitlinear_forward_plan; out[4] = 2 with out[5] =
 * K tiles per wave for the register form, out[4] = 1 with out[5] = dynamic LDS bytes
 * for the LDS form, or out[4] = 4 with out[5] = K tiles per wave for the 5..16-token LDS
 * form); otherwise the activation quantiser runs first and out[] describes
 * the forward launch exactly as bitlinear_forward_plan.  Returns BL_OK,
 * BL_ERR_INVALID_ARG (as bitlinear_forward_plan) or BL_ERR_UNSUPPORTED (dt).
 */
int bitlinear_forward_fused_plan(int64_t M, int64_t N, int64_t K, int dt, int32_t out[6]);

/*
 * Measurement probes: not steps of the method, the ceilings a benchmark holds the
 * kernels above against.
 *
 * bitlinear_probe_stream reads `bytes` (a multiple of 1024, at least 1024) of device
 * memory at `buf` (16-byte aligned) with the decode kernels' access pattern (1 KiB tiles,
 * 16 bytes per lane, non-temporal, each wave's 8-tile run in flight at once) and does no
 * other work.  out[i] (device, uint32, out_words >= bitlinear_probe_stream_words(bytes))
 * receives the XOR of the 32-bit words of the i-th 32 KiB block (the last block may be
 * shorter).  bitlinear_probe_stream_words returns -1 for an invalid size.
 *
 * bitlinear_probe_read reads `bytes` (a multiple of 16, at least 16) of device memory at
 * `buf` (16-byte aligned) with a plain grid-stride loop: `workgroups` (1 .. 2^20) of 256
 * lanes, lane i of the grid taking the 16-byte words i, i + S, i + 2S, ... (S = 256 x
 * workgroups), eight loads in flight per lane, non-temporal when `nontemporal` is 1 (0:
 * ordinary loads).  It shares no access pattern with the BitLinear kernels: the plain HBM
 * read ceiling for a launch of that size.  out[workgroups] (device, uint32) receives, per
 * workgroup, the XOR of the 32-bit words it read.
 *
 * bitlinear_probe_mfma runs `workgroups` x 4 waves, each issuing 16 independent
 * v_mfma_i32_16x16x64_i8 per iteration for `iters` iterations (32768 int8 operations
 * each), with no memory traffic; out[workgroups] (device) receives checksums.
 */
int64_t bitlinear_probe_stream_words(int64_t bytes);
int bitlinear_probe_stream(const void* buf, int64_t bytes, uint32_t* out, int64_t out_words, void* stream);
int bitlinear_probe_read(const void* buf, int64_t bytes, int64_t workgroups, int nontemporal, uint32_t* out,
                         void* stream);
int bitlinear_probe_mfma(int64_t iters, int64_t workgroups, uint32_t* out, void* stream);
/*
 * bitlinear_probe_prefill_occupancy writes to out[4] (host memory) the workgroups per
 * compute unit that the HIP runtime reports as resident at once for the one-group prefill
 * kernels: 64 x 256 and 64 x 192 tiles of bitlinear_forward, then the same two of
 * bitlinear_forward_ws's split-tail form.  The planner of bitlinear_forward_ws assumes 3
 * and 4.  Needs a current HIP device; BL_ERR_HIP if the query fails.
 */
int bitlinear_probe_prefill_occupancy(int32_t out[4]);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H_ */
