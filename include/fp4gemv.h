/*
 * fp4gemv.h -- C ABI of the MI355X (gfx950) decode matrix-vector library for
 * block-scaled 4-bit and FP8 weights.
 *
 * What the library computes.  Decoding one token passes its hidden state through
 * every weight matrix once; a matrix with d_out rows and d_in columns turns a
 * length-d_in vector into a length-d_out one at two flops per weight while all
 * of its bytes stream from memory, so the step time is set by bytes read over
 * achieved bandwidth (mdjawad.com DGX Spark feed, section "Decode speed is bytes
 * divided by bandwidth").  Every entry point here computes, for M input vectors
 * x_m (bf16) and a dequantised weight matrix w,
 *
 *     y[m][r] = sum_k w[r][k] * x_m[k]            (FP32 accumulation)
 *
 * where w is reconstructed from one of three formats:
 *   FP4G_NVFP4   E2M1 element x E4M3 scale of its 16-weight block x one FP32
 *                tensor scale (same feed, section "Fewer bytes per weight: NVFP4";
 *                the formula was lost in extraction and is read as a product).
 *   FP4G_MXFP4   E2M1 element x E8M0 (power of two) scale of its 32-weight block
 *                (magicnetworld.com Ling-3.0 MoE decode article, sec. 3 and its
 *                glossary name MXFP4 for the MoE experts; the block size of 32 is
 *                the reading taken here).
 *   FP4G_FP8_ROW OCP E4M3FN element x one FP32 scale per row (the FP8 output
 *                layer of the same article, sec. 7, and of the feed).
 * E2M1 is 1 sign, 2 exponent (bias 1), 1 mantissa bit; its values are 0, +-0.5,
 * +-1, +-1.5, +-2, +-3, +-4, +-6.  E4M3FN has bias 7, no infinities, and
 * S.1111.111 as NaN.  E8M0 is 2^(e-127) with 0xFF as NaN.
 *
 * M = 1 is batch-1 decode; M in 2..8 is the verify pass of speculative decoding,
 * which multiplies each matrix by K+1 vectors at fixed bytes (feed, section
 * "More tokens per weight read").
 *
 * Conventions for every function below:
 *  - Pointers named *_dev are device pointers (HBM); pointers to descriptors and
 *    to status outputs named *_host are host pointers.  The caller owns every
 *    buffer; the library allocates nothing and keeps no mutable global state.
 *  - All device work is enqueued asynchronously on `stream` (a hipStream_t passed
 *    as void*; NULL is the default stream).  Nothing synchronises.
 *  - Every argument is validated on the host before any HIP call; a function that
 *    returns an error has enqueued nothing.  No C++ exception crosses the ABI.
 *    The library loads, and its validation runs, on a machine without a GPU.
 *  - Formats are never reinterpreted: a descriptor whose format or layout tag
 *    does not match what the entry point accepts is refused with FP4G_E_FORMAT
 *    (the article's sec. 11 describes FP8 weights silently read as BF16; this
 *    library refuses instead of guessing).
 *  - Outputs are overwritten, never accumulated into, and must not overlap any
 *    input or each other (FP4G_E_ALIAS).
 *  - Floating-point results are the exact sum up to FP32 rounding in an
 *    unspecified but fixed order: repeated calls with the same inputs and shapes
 *    give bit-identical outputs.
 */
#ifndef FP4GEMV_H
#define FP4GEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4G_ABI_VERSION 1u

/* Layout tag written by fp4g_pack into every descriptor it fills in.  Kernels
 * refuse any other tag. */
#define FP4G_LAYOUT_TILE64x256 0x46344731u

typedef enum {
  FP4G_OK = 0,
  FP4G_E_NULL = 1,      /* a required pointer is NULL */
  FP4G_E_SHAPE = 2,     /* bad d_out, d_in, M, expert counts, or buffer too small */
  FP4G_E_ALIGN = 3,     /* packed not 256-B aligned, or a vector not 16-B aligned */
  FP4G_E_FORMAT = 4,    /* wrong format for this call, unknown layout tag, bad scale */
  FP4G_E_WORKSPACE = 5, /* ws_bytes smaller than fp4g_workspace_bytes() */
  FP4G_E_PATH = 6,      /* the requested kernel path does not exist for this call */
  FP4G_E_ALIAS = 7,     /* an output overlaps an input or another output */
  FP4G_E_HIP = 8        /* the HIP runtime reported an error at launch */
} fp4g_status;

typedef enum { FP4G_NVFP4 = 1, FP4G_MXFP4 = 2, FP4G_FP8_ROW = 3 } fp4g_format;

/* Kernel path of the NVFP4/MXFP4 products.  VALU: one v_dot2 per weight pair and
 * vector.  MFMA: the products on the matrix cores (bf16 MFMA on exact bf16
 * weights; block scales applied per block in FP32).  AUTO takes MFMA from M = 3
 * on and VALU below.  The VALU kernel takes up to 8 vectors, the MFMA kernel up
 * to 16 (FP4G_MAX_M_WIDE: a verify block of up to 15 drafts, feed section "More
 * tokens per weight read"); VALU with more than 8 NVFP4/MXFP4 vectors is
 * FP4G_E_PATH.  FP8 rows have only the VALU kernel, up to 16 vectors for plain
 * products and the greedy pick (8 for a fused gate/up pair): MFMA is refused
 * there with FP4G_E_PATH.  Both paths give
 * the same results up to the order of the FP32 additions.
 * A8 (W4A8; fp4_skinny_gemm, fp4_gemv_grouped and fp4_gate_up_silu on MXFP4
 * weights only, M in 1..16, else FP4G_E_PATH): the input is first quantised per
 * vector and 32 columns to E4M3 with an E8M0 scale, the smallest 2^e with
 * amax / 2^e <= 448, round to nearest even (the Ling-3.0 article measures MXFP4
 * experts with 8-bit activations, sec. 5-6); the product of those activations
 * is then exact up to the order of the FP32 additions (scaled FP4 x FP8 matrix
 * cores).  x must be finite on this path. */
typedef enum { FP4G_PATH_AUTO = 0, FP4G_PATH_VALU = 1, FP4G_PATH_MFMA = 2, FP4G_PATH_A8 = 3 } fp4g_path;

/* Operation ids for fp4g_workspace_bytes. */
typedef enum {
  FP4G_OP_GEMV = 1,     /* fp4_gemv and fp4_skinny_gemm; desc = fp4g_weight */
  FP4G_OP_GATE_UP = 2,  /* fp4_gate_up_silu; desc = fp4g_weight (gate) */
  FP4G_OP_MOE = 3,      /* moe_route_gemv; desc = fp4g_moe */
  FP4G_OP_LMHEAD = 4,   /* fp8_lmhead_gemv; desc = fp4g_weight */
  FP4G_OP_GROUPED = 5,  /* fp4_gemv_grouped; desc = fp4g_group */
  FP4G_OP_LMHEAD_ARGMAX = 6  /* fp8_lmhead_argmax; desc = fp4g_weight */
} fp4g_op;

/* Most matrices one fp4_gemv_grouped call takes. */
#define FP4G_MAX_GROUP 4
/* Vectors per call: 1..FP4G_MAX_M_WIDE, except the VALU path of the
 * NVFP4/MXFP4 products and the FP8 gate/up pair (1..FP4G_MAX_M). */
#define FP4G_MAX_M 8
#define FP4G_MAX_M_WIDE 16

/* A packed weight matrix.  A plain view: it owns nothing.  Filled in by
 * fp4g_pack; callers must not edit it. */
typedef struct {
  uint32_t format;      /* fp4g_format */
  uint32_t layout_tag;  /* FP4G_LAYOUT_TILE64x256 */
  int32_t d_out;        /* rows, >= 1 */
  int32_t d_in;         /* columns, >= 32 and a multiple of 32 */
  const void* packed;   /* device, 256-B aligned, fp4g_packed_bytes() bytes */
  uint64_t packed_bytes;
  float tensor_scale;   /* NVFP4: finite, multiplies every weight; other formats: 1.0 */
  uint32_t reserved;
} fp4g_weight;

/* A mixture-of-experts layer (article sec. 3: each token is routed to top_k of
 * num_experts routed experts, plus one shared expert).  Routed expert e's
 * matrices are gate / up / down with their `packed` pointer advanced by
 * e * stride_* bytes; the three descriptors describe expert 0.  Every expert of
 * one kind has the same format, shape and tensor scale.  gate and up are
 * d_ff x hidden; down is hidden x d_ff. */
typedef struct {
  int32_t num_experts;  /* 1..1024 */
  int32_t top_k;        /* 1..8 and <= num_experts */
  int32_t hidden;
  int32_t d_ff;
  fp4g_weight gate, up, down;
  uint64_t stride_gate, stride_up, stride_down; /* bytes, multiples of 256 */
  int32_t has_shared;   /* 0 or 1 */
  int32_t act;          /* FP4G_ACT_BF16, or FP4G_ACT_MXFP8 (MXFP4 experts only) */
  fp4g_weight sh_gate, sh_up, sh_down;          /* used when has_shared == 1 */
} fp4g_moe;

/* Activations of a MoE layer.  BF16: the products take x and h as bf16.
 * MXFP8 (W4A8, the Ling-3.0 article's measured configuration, Table 1 and
 * sec. 3): x and each expert's bf16 h are quantised per vector and 32 columns to
 * E4M3 with an E8M0 scale as FP4G_PATH_A8 does, and the products run on the
 * scaled FP4 x FP8 matrix cores; other values are FP4G_E_PATH, and so is MXFP8
 * with NVFP4 experts. */
#define FP4G_ACT_BF16 0
#define FP4G_ACT_MXFP8 1

/* Matrices that multiply the same input: the query, key and value projections of
 * an attention layer, all read by one decode step (feed, section "Decode speed is
 * bytes divided by bandwidth").  All members share format (NVFP4 or MXFP4) and
 * d_in; d_out may differ.  Only w[0..n) are read. */
typedef struct {
  int32_t n;            /* 1..FP4G_MAX_GROUP */
  int32_t reserved;
  fp4g_weight w[FP4G_MAX_GROUP];
} fp4g_group;

/* --- library info ------------------------------------------------------- */

uint32_t fp4g_abi_version(void);

/* Static string for a status code; never NULL. */
const char* fp4g_status_string(int32_t status);

/* --- packing (load time) -------------------------------------------------- */

/* Bytes of the packed image of a d_out x d_in matrix of `format`, or 0 if the
 * shape is invalid.  Rows are padded to 64 and columns to 256.  NVFP4 spends
 * 4.5 bits per weight (4-bit element plus an 8-bit scale per 16; feed, section
 * "Fewer bytes per weight: NVFP4"), MXFP4 4.25, FP8_ROW 8 plus 4 bytes per row.
 *
 * Packed layout (FP4G_LAYOUT_TILE64x256).  Let R = ceil(d_out/64) row groups
 * and C = ceil(d_in/256) column chunks.  Tile (g, c), for 0 <= g < R and
 * 0 <= c < C, starts at byte (g*C + c) * T.  Inside a tile, lane l (0..63)
 * stands for row 64g + l:
 *   NVFP4 (T = 9216): for slot j in 0..7, bytes j*1024 + 16l .. +15 hold the
 *     logical code bytes of columns 256c + 32j .. +31 of that row (byte b holds
 *     column 2b in bits 0-3, 2b+1 in bits 4-7); bytes 8192 + 16l .. +15 hold the
 *     E4M3 scales of that row's blocks 16c .. 16c+15.
 *   MXFP4 (T = 8704): codes as NVFP4; bytes 8192 + 8l .. +7 hold the E8M0 scales
 *     of blocks 8c .. 8c+7.
 *   FP8_ROW (T = 16384): for slot j in 0..15, bytes j*1024 + 16l .. +15 hold the
 *     codes of columns 256c + 16j .. +15.  After the R*C tiles follow R*64 FP32
 *     row scales.
 * Padding rows and columns hold zero bytes. */
uint64_t fp4g_packed_bytes(uint32_t format, int32_t d_out, int32_t d_in);

/* Pack a logical matrix into `packed_dev`.
 *   codes_dev   NVFP4/MXFP4: u8[d_out][d_in/2], byte j of a row holds column 2j in
 *               bits 0-3 and column 2j+1 in bits 4-7.  FP8_ROW: u8[d_out][d_in].
 *   scales_dev  NVFP4: u8[d_out][d_in/16] E4M3; MXFP4: u8[d_out][d_in/32] E8M0;
 *               FP8_ROW: f32[d_out].
 *   packed_dev  256-B aligned, packed_bytes >= fp4g_packed_bytes(...).
 *   out_host    receives the descriptor.
 * A pure byte permutation: fp4g_unpack restores the inputs bit for bit.  NaN
 * scale codes are not checked here; see fp4g_validate. */
int32_t fp4g_pack(uint32_t format, int32_t d_out, int32_t d_in, const void* codes_dev,
                  const void* scales_dev, float tensor_scale, void* packed_dev,
                  uint64_t packed_bytes, fp4g_weight* out_host, void* stream);

/* Quantise a bf16 matrix w_dev [d_out][d_in] (d_in % 32 == 0; finite values) into
 * the logical codes and scales fp4g_pack takes (feed, section "Fewer bytes per
 * weight: NVFP4": each block's largest magnitude maps to 6, the E2M1 maximum;
 * E4M3 block scales; one FP32 tensor scale bringing them into E4M3's range):
 *   NVFP4:   s_T = amax(w) / (6 * 448) (1 if all zero); block scale code =
 *            E4M3(amax_block / (6 s_T)); element = E2M1(w / (s_block * s_T)),
 *            0 where the block scale is 0.
 *   MXFP4:   per 32 weights the smallest power of two 2^e with amax/2^e <= 6,
 *            E8M0 code e + 127 (clamped to 0..254; 127 for an all-zero block);
 *            element = E2M1(w / 2^e).
 *   FP8_ROW: per row s = amax_row / 448 (1 if all zero) as the FP32 row scale;
 *            element = E4M3(w / s).
 * Rounding: nearest, ties to the even code, saturating (E2M1 at 6, E4M3 at 448);
 * a value that rounds to zero gets the +0 code.  s_T and s are the FP32 values
 * nearest to their quotients; every code is the grid value nearest to the exact
 * quotient of the bf16 input and the stored FP32 scales (no intermediate
 * rounding decides a code).
 *   codes_dev   NVFP4/MXFP4: u8[d_out][d_in/2]; FP8_ROW: u8[d_out][d_in].
 *   scales_dev  u8[d_out][d_in/16] (NVFP4), u8[d_out][d_in/32] (MXFP4), f32[d_out].
 *   tensor_scale_dev  NULL or one f32: s_T (NVFP4), 1.0 otherwise.
 *   ws_dev      NVFP4 only: >= 256 bytes of scratch (any contents); else unused. */
int32_t fp4g_quantize(uint32_t format, int32_t d_out, int32_t d_in, const uint16_t* w_dev, void* codes_dev,
                      void* scales_dev, float* tensor_scale_dev, void* ws_dev, uint64_t ws_bytes, void* stream);

/* Inverse of fp4g_pack: write the logical codes and scales of W (the formats as
 * the pages define them: feed, section "Fewer bytes per weight: NVFP4"; Ling-3.0
 * article, glossary (MXFP4) and sec. 7 (the FP8 output layer)).  A pure byte
 * permutation, so a pack/unpack round trip is bit-exact. */
int32_t fp4g_unpack(const fp4g_weight* W_host, void* codes_dev, void* scales_dev, void* stream);

/* Count, into the device int64 at *bad_dev, the scale entries of W that are NaN
 * codes (E4M3 S.1111.111, E8M0 0xFF) or non-finite FP32 row scales.  Callers
 * check it once at load time; the product kernels never test scales.  (The
 * Ling-3.0 article, sec. 11, describes weights silently taken in the wrong
 * format and a service that only got slower; this check and the descriptors'
 * format and layout tags are the guard against the same with bad scales.) */
int32_t fp4g_validate(const fp4g_weight* W_host, int64_t* bad_dev, void* stream);

/* --- workspace ---------------------------------------------------------------- */

/* Bytes of device workspace the call `op` needs for descriptor `desc_host`
 * (fp4g_weight, fp4g_group or fp4g_moe, see fp4g_op) and M vectors; 0 means none
 * (then ws_dev may be NULL).  A call given less returns FP4G_E_WORKSPACE.  The
 * workspace holds split-K exchange slots, the greedy pick's running maxima and
 * (moe_route_gemv) routing tables and intermediate vectors.  The caller
 * zero-fills a workspace once, before its first use; every call leaves the slots
 * and maxima at zero again when its kernels complete, so one zero-filled
 * workspace (of the largest size needed) serves calls of any shape.  A slot
 * left non-zero (a workspace never zero-filled, or a call interrupted, or two
 * calls overlapping on it) would be taken as a partner's partial sum:
 * fp4g_workspace_check finds such slots before a call.  moe_route_gemv is the exception: it also keeps its
 * routing tables and intermediate vectors in the workspace, after the slots, so
 * its workspace may be shared only by moe_route_gemv calls on layers of one
 * shape (any M), and by nothing else.  Calls that share a workspace must be
 * ordered on one stream.  Returns 0 also for invalid arguments. */
uint64_t fp4g_workspace_bytes(int32_t op, const void* desc_host, int32_t M);

/* Count, into *nonzero_host, the 8-byte words of the part of ws_dev that must
 * be zero before the call (op, desc_host, M): the exchange slots and running
 * maxima (for FP4G_OP_MOE the slots only, not the tables after them).  0 means
 * the call may use the workspace; a caller that gets more must zero-fill it
 * (or refuse the call).  Synchronises `stream`; meant for load time, tests and
 * debugging, not for the decode loop.  Errors: FP4G_E_NULL, FP4G_E_SHAPE (no
 * workspace needed, or a bad descriptor), FP4G_E_WORKSPACE (ws_bytes smaller
 * than fp4g_workspace_bytes), FP4G_E_ALIGN (ws_dev not 256-B aligned). */
int32_t fp4g_workspace_check(int32_t op, const void* desc_host, int32_t M, const void* ws_dev,
                             uint64_t ws_bytes, uint64_t* nonzero_host, void* stream);

/* --- products --------------------------------------------------------------- */

/* y_dev[r] = sum_k w[r][k] * x_dev[k] for an NVFP4 or MXFP4 matrix (M = 1, the
 * batch-1 decode GEMV whose speed is the bytes of W over the memory bandwidth:
 * feed, section "Decode speed is bytes divided by bandwidth").  x_dev: bf16 bit
 * patterns [d_in], 16-B aligned.  y_dev: f32 [d_out], 16-B aligned. */
int32_t fp4_gemv(const fp4g_weight* W_host, const uint16_t* x_dev, float* y_dev, void* ws_dev,
                 uint64_t ws_bytes, void* stream);

/* Y_dev[m][r] = sum_k w[r][k] * X_dev[m][k] for m < M, M in 1..16 (the verify
 * product of speculative decoding; above 8 on the matrix-core path only).  X_dev: bf16 [M][d_in]; Y_dev: f32 [M][d_out].
 * path: fp4g_path. */
int32_t fp4_skinny_gemm(const fp4g_weight* W_host, const uint16_t* X_dev, int32_t M, float* Y_dev,
                        int32_t path, void* ws_dev, uint64_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): fp4_skinny_gemm with
 * the split-K workspace taken from a fixed device array inside the library
 * instead of ws_dev.  Same arguments, kernels and results as fp4_skinny_gemm
 * (bit for bit, same plan).  The array holds FP4G_NOALLOC_SCRATCH_BYTES; a call
 * whose fp4g_workspace_bytes(FP4G_OP_GEMV, W, M) exceeds it returns
 * FP4G_E_WORKSPACE (every dense product of the feed's model fits up to M = 16:
 * the largest, 5120 x 17408, needs 5 MiB).  Each GPU holds one array until the
 * process ends, shared by every call on that GPU: it starts zero-filled and
 * every call leaves it as it found it, so calls must be ordered (one stream, or
 * streams synchronised with each other); calls that overlap in time on one GPU
 * race on it and give unspecified results.  The first call on a device looks up
 * the array's address there (a HIP call that allocates nothing); nothing calls
 * hipMalloc, hipFree or any allocating routine. */
#define FP4G_NOALLOC_SCRATCH_BYTES (16ull << 20)
int32_t fp4_skinny_gemm_noalloc(const fp4g_weight* W_host, const uint16_t* X_dev, int32_t M, float* Y_dev,
                                int32_t path, void* stream);

/* Several products of one input in one launch: Y_dev[i][m][r] = sum_k
 * w_i[r][k] * X_dev[m][k] for each member i of G, m < M in 1..16 (above 8 on
 * the matrix-core path only).  Members share format and d_in: NVFP4 or MXFP4,
 * or FP8_ROW with each member's own row scales (the FP8 projections of a mixed
 * layout; VALU path, M in 1..16).  X_dev: bf16 [M][d_in]; Y_dev: host array of
 * G->n device pointers, each f32 [M][w_i.d_out], 16-B aligned and disjoint.
 * path: fp4g_path.  Each member's results are those of fp4_skinny_gemm (FP8:
 * fp8_lmhead_gemv) on it alone up to the order of the FP32 additions. */
int32_t fp4_gemv_grouped(const fp4g_group* G_host, const uint16_t* X_dev, int32_t M,
                         float* const* Y_host, int32_t path, void* ws_dev, uint64_t ws_bytes, void* stream);

/* Fused MLP front half: g = Wg X_m, u = Wu X_m, H_dev[m][r] = bf16_rne(SiLU(g[r]) *
 * u[r]) with SiLU(z) = z / (1 + e^-z), for m < M in 1..16 (above 8 on the
 * matrix-core path only).  Wg and Wu are NVFP4 or MXFP4 matrices of one shape
 * d_ff x hidden (feed, section "Decode speed is bytes divided by bandwidth":
 * gate and up projections are 17408 x 5120 in the dense model), or two FP8_ROW
 * matrices, each with its own row scales (the FP8 MLPs of the last layers in the
 * feed's mixed checkpoint, section "Fewer bytes per weight: NVFP4"; VALU path,
 * M in 1..8).  With FP4G_PATH_A8 (MXFP4 pairs) g and u are the W4A8 products of
 * the input quantised once for both.  X_dev: bf16 [M][hidden]; H_dev: bf16
 * [M][d_ff]. */
int32_t fp4_gate_up_silu(const fp4g_weight* Wg_host, const fp4g_weight* Wu_host,
                         const uint16_t* X_dev, int32_t M, uint16_t* H_dev, int32_t path,
                         void* ws_dev, uint64_t ws_bytes, void* stream);

/* One MoE layer for M in 1..16 tokens (article sec. 3 and the sec. 4 flowchart:
 * route to top_k of num_experts, read only the chosen experts, accumulate back to
 * the hidden size; sec. 8 notes that M tokens touch the union of their experts).
 * Per token m:
 *   ids   = the top_k experts by logits_dev[m][:], in descending logit order,
 *           equal logits ordered by the lower index;
 *   g_j   = softmax over the top_k selected logits;
 *   d_e   = down_e( bf16_rne( SiLU(gate_e x_m) * (up_e x_m) ) );
 *   Y[m]  = sum_j g_j d_{ids_j} + d_shared      (d_shared only if has_shared).
 * Only the union of the M tokens' experts is read from memory; routing never
 * leaves the device.  Two launches for M = 1, 2 (every gate/up workgroup routes
 * the tokens itself); three from M = 3 on (routing once, gate/up on the matrix
 * cores, then down: on the VALU up to M = 4, on the matrix cores from M = 5;
 * verify blocks of 9..16 tokens the same way, e.g. the feed's 11 positions in
 * section "DFlash2: drafting a block in one pass").
 *   X_dev       bf16 [M][hidden];  logits_dev f32 [M][num_experts];
 *   Y_dev       f32  [M][hidden];
 *   topk_ids_dev i32 [M][top_k];  topk_w_dev f32 [M][top_k];
 *   H_dev       optional (NULL allowed) bf16 [M][top_k + has_shared][d_ff]: the
 *               intermediate of each (token, chosen expert), shared expert last. */
int32_t moe_route_gemv(const fp4g_moe* moe_host, const uint16_t* X_dev, const float* logits_dev,
                       int32_t M, float* Y_dev, int32_t* topk_ids_dev, float* topk_w_dev,
                       uint16_t* H_dev, void* ws_dev, uint64_t ws_bytes, void* stream);

/* FP8 output layer (article sec. 7; feed, section "MTP: the drafter inside the
 * checkpoint" -- the layer scores the whole vocabulary): logits_dev[m][r] =
 * s_row[r] * sum_k e4m3(c[r][k]) * X_dev[m][k] for M in 1..16 (a verify block
 * of up to 15 drafts is scored with one read of the layer: feed, section "DFlash2:
 * drafting a block in one pass", verifies 11 positions).  W must be FP8_ROW.
 * X_dev: bf16 [M][d_in]; logits_dev: f32 [M][d_out]. */
int32_t fp8_lmhead_gemv(const fp4g_weight* W_host, const uint16_t* X_dev, int32_t M,
                        float* logits_dev, void* ws_dev, uint64_t ws_bytes, void* stream);

/* Greedy pick from the FP8 output layer in the same launch (the layer scores
 * the vocabulary and decoding keeps its best token: feed, sections "MTP: the
 * drafter inside the checkpoint" and "Shaving the step"), over the rows
 * [row_begin, row_begin + n_rows) -- the whole vocabulary, or a draft head that
 * scores a leading part of it.  For m < M in 1..16:
 *   logit[m][r] = s_row[r] * sum_k e4m3(c[r][k]) * X_dev[m][k] as fp8_lmhead_gemv,
 *   top_idx_dev[m] = the row r (absolute, row_begin <= r < row_begin + n_rows)
 *     with the largest FP32 logit, the lower row on equal logits (-0 == +0),
 *   top_val_dev[m] = that logit.
 * row_begin % 64 == 0.  logits_dev: NULL, or f32 [M][n_rows] (logit of row
 * row_begin + j at j).  top_idx_dev i32 [M], top_val_dev f32 [M].  The workspace
 * (fp4g_workspace_bytes(FP4G_OP_LMHEAD_ARGMAX, ...), a few KiB) must be
 * zero-filled once; every call leaves it at zero.  One workgroup per 64 rows (no
 * split-K), then a one-wave launch that collects the pick. */
int32_t fp8_lmhead_argmax(const fp4g_weight* W_host, const uint16_t* X_dev, int32_t M, int32_t row_begin,
                          int32_t n_rows, float* logits_dev, int32_t* top_idx_dev, float* top_val_dev,
                          void* ws_dev, uint64_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4GEMV_H */
