/*
 * rb.h -- C ABI of librb: residual binarized weights on AMD Instinct MI355X (gfx950).
 *
 * The library derives k residual sign bit-planes with dual scales from a full
 * precision weight matrix, and runs the matmul-free product on the packed planes,
 * plus the binary-codebook (sub-1-bit) variant. Every entry point only validates its
 * arguments on the host and enqueues kernels on the caller's stream: no allocation,
 * no free, no synchronisation, no exceptions across the ABI.
 *
 * Sources (web pages on the method, cited by title and section):
 *   [RaBiT] "RaBiT: Residual-Aware Binarization Training for Accurate and Efficient
 *           LLMs" (paper summary page): background "Residual binarization", sections
 *           "Method step details" (Algorithm 2) and "Technical novelty".
 *   [BTC]   "亚1比特大模型量化技术突破与实践" (BTC-LLM binary codebook page):
 *           sections 2.1.1, 2.1.2, 3.2.1, 3.2.2, 5.1, 5.2.
 *   [SigmoidBitLinear] the SigmoidBitLinear blog page ({0, scale_row} weights).
 *
 * Conventions shared by every call
 *   - Matrices are row-major. W is N x K (output x input), y = W x.
 *   - Every pointer except the host-side helpers' is a DEVICE pointer owned by the
 *     caller (memory from hipMalloc / torch); the library keeps no pointer after a
 *     call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). The work
 *     is only enqueued; results are ready when the stream reaches that point.
 *   - Host-detectable errors (bad sizes, NULL pointers, misalignment, workspace too
 *     small, unsupported dtype) are returned synchronously before anything is
 *     enqueued. RB_ERR_HIP means a launch failed (hipGetLastError after launch).
 *   - Calls are stateless and may be made from several host threads; calls that share
 *     an output or a workspace buffer must be ordered by the caller (same stream).
 *
 * Bit-plane format ("planes"): k planes, each N rows of `ldp` uint32 words
 *   (ldp >= ceil(K/32)), plane stride N*ldp words. Bit j of word w of row n is column
 *   32*w + j (LSB first); bit 1 means +1, bit 0 means -1; sign(0) = +1 (also -0.0).
 *   Bits for columns >= K are 0. Words ceil(K/32) .. ldp-1 are padding: never read,
 *   never written. [RaBiT "Technical novelty": 32 columns per uint32]
 * Scales: g is [k][N] (one per output row and plane), h is [k][K] (one per input
 *   column and plane), both in `scale_dtype`; W_hat = sum_i g_i (.) B_i (.) h_i.
 *   [RaBiT "Residual binarization"]
 */
#ifndef RB_H_
#define RB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rb_status {
  RB_OK = 0,
  RB_ERR_INVALID_ARG = 1,  /* a size, enum or pointer is out of range / NULL          */
  RB_ERR_UNSUPPORTED = 2,  /* a valid combination this build does not implement      */
  RB_ERR_MISALIGNED = 3,   /* a pointer violates the alignment the entry point states */
  RB_ERR_WORKSPACE = 4,    /* ws is NULL or ws_bytes < rb_workspace_bytes(...)        */
  RB_ERR_HIP = 5           /* a kernel launch failed                                  */
} rb_status;

typedef enum rb_dtype { RB_F32 = 0, RB_F16 = 1, RB_BF16 = 2 } rb_dtype;

typedef enum rb_op {
  RB_OP_PACK = 0,
  RB_OP_GEMV = 1,
  RB_OP_GEMM_SMALL = 2,
  RB_OP_CODEBOOK_ENCODE = 3,
  RB_OP_CODEBOOK_GEMV = 4,
  RB_OP_SVID_INIT = 5,
  RB_OP_QAT_BACKWARD = 6
} rb_op;

/* Version of this ABI (major*10000 + minor*100 + patch). */
int rb_version(void);

/* Static string naming a status code; never NULL. */
const char* rb_status_string(rb_status s);

/* Device workspace (bytes) an operation needs for the given sizes; 0 when it needs
 * none. Every workspace begins with a zero region of ceil(8N / 256) * 256 bytes (one
 * 64-bit accumulator per output row), which rb_gemv and rb_gemv_variant need all-zero on
 * entry and return to all-zero before their last kernel ends; the bytes after it are
 * scratch. rb_gemm_small, rb_svid_init and rb_qat_backward use only bytes after the zero
 * region and never write it. So: zero-fill a workspace once after allocation, and one
 * buffer of the largest size its calls need can serve all of them (calls on one stream;
 * calls that overlap in time need separate workspaces). */
size_t rb_workspace_bytes(rb_op op, int32_t k, int64_t N, int64_t K, int64_t M);

/* Storage cost in bits per weight of k planes plus per-row g_i and (if has_h)
 * per-column h_i in scale_dtype: k + bits(scale_dtype) * k * (N + has_h*K) / (N*K).
 * With N = K = 4096, k = 2 and fp16 scales this is 2.015625, the "2.02 effective
 * bits" of [RaBiT "Limitations"]. Returns -1 on invalid arguments. */
double rb_storage_bits_per_weight(int64_t N, int64_t K, int32_t k, rb_dtype scale_dtype,
                                  int32_t has_h);

/*
 * rb_pack -- derive k residual sign planes and their scales from W.
 *   [RaBiT "Method step details", Algorithm 2 forward pass; deployment derives the
 *   planes once and freezes them]
 *     R_0 = W;  for i = 0..k-1:  B_i = sign(R_i)            (sign(0) = +1)
 *                                g_i = sum|R_i| h_i / sum h_i^2, rounded to nearest-even
 *                                      in scale_dtype (row mean |R_i| when h = 1)
 *                                R_{i+1} = R_i - g_i (.) B_i (.) h_i   (stored g_i)
 *   The sums are taken in fp64 and the residual is kept in fp64, so the result equals
 *   the exact derivation except for scales whose quotient falls within ~K*2^-53
 *   (relative) of a rounding midpoint, which may round to either neighbour.
 *
 *   W        [N][ldw] elements of w_dtype (RB_F32, RB_F16 or RB_BF16), 4-byte aligned
 *   N, K     rows (outputs) and columns (inputs); 1 <= N, K < 2^31
 *   ldw      row stride of W in elements, >= K
 *   k        number of planes, 1..4
 *   group    0: one scale per row (g is [k][N]); otherwise a power of two in 2..64:
 *            one scale per `group` consecutive columns (g is [k][N][ceil(K/group)]),
 *            mean |R| over the group's columns; requires h == NULL
 *   h        [k][K] in scale_dtype, or NULL for all ones
 *   scale_dtype  RB_F16 or RB_F32 (type of g and h)
 *   planes   output, [k][N][ldp] uint32, 16-byte aligned; ldp >= ceil(K/32)
 *   g        output scales, scale_dtype, layout above
 *   d_status optional device int32; the call ORs 1 into it if W holds a NaN or an
 *            infinity (outputs are then unspecified). NULL to skip the check report.
 */
rb_status rb_pack(const void* W, rb_dtype w_dtype, int64_t N, int64_t K, int64_t ldw, int32_t k,
                  int32_t group, const void* h, rb_dtype scale_dtype, uint32_t* planes, int64_t ldp,
                  void* g, int32_t* d_status, void* stream);

/*
 * rb_gemv -- the matmul-free product on packed planes for decode-sized batches.
 *   [RaBiT "Residual binarization": the k paths run in parallel with additions and
 *   element-wise scaling only]
 *     y[m][n] = sum_i g_i[n] * sum_c B_i[n][c] * h_i[c] * x[m][c]
 *   computed as sum_i g_i[n] * (2*T_i[m][n] - S_i[m]) with T_i the sum of h_i (.) x over
 *   the columns whose bit is 1 and S_i the sum over all columns (fp32 accumulation),
 *   then rounded to y_dtype.
 *
 *   planes, ldp   as produced by rb_pack (16-byte aligned)
 *   g, h          [k][N] and [k][K] (h may be NULL = ones) in scale_dtype (F16 or F32)
 *   k             1..4;  N, K >= 1
 *   x             [M][K] in x_dtype (RB_F16 or RB_F32), 16-byte aligned
 *   M             1..16 (larger batches: rb_gemm_small)
 *   y             output [M][N] in y_dtype (RB_F16 or RB_F32), 16-byte aligned
 *   ws, ws_bytes  device workspace of at least rb_workspace_bytes(RB_OP_GEMV, k, N, K, M)
 *                 bytes (the same for every M), zero-filled once after allocation; its first
 *                 part is left zero by every call, the rest holds per-call partial sums
 *   A batch of M >= 4 rows (M = 3 when K >= 2N or N >= 2K; M >= 2 when k*N*K >= 2^27) with fp16 x, K a multiple of 64, an
 *   even ldp and h NULL or fp16 and 16-byte aligned is computed as rb_gemm_small computes it
 *   (on the matrix cores, fp32 accumulation); other calls on the vector units. Either way
 *   the result meets the same bound against the exact product.
 */
rb_status rb_gemv(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                  rb_dtype scale_dtype, int32_t k, int64_t N, int64_t K, const void* x,
                  rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* ws, size_t ws_bytes,
                  void* stream);

/*
 * rb_gemv_noalloc -- rb_gemv for callers that cannot allocate device memory: code under HIP
 *   graph capture, tight serving loops, harnesses that forbid hipMalloc. Same product, same
 *   arguments and errors as rb_gemv, except that there is no ws / ws_bytes: the workspace is a
 *   fixed 4 MB array inside the library, one per GPU, held from the library's load until the
 *   process ends (the call itself allocates nothing). Its device address is looked up once per
 *   device. Each call first clears the array's zero region (one small fill kernel on `stream`,
 *   no memset) and then runs rb_gemv's kernels on it.
 *   Returns RB_ERR_WORKSPACE when rb_workspace_bytes(RB_OP_GEMV, k, N, K, M) exceeds 4 MB
 *   (e.g. more than 524288 rows), before touching the device.
 *   All calls on one GPU share its array: calls that overlap in time on one GPU (different
 *   streams, threads or processes without ordering) race and give undefined results; order
 *   them on one stream.
 */
rb_status rb_gemv_noalloc(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                          rb_dtype scale_dtype, int32_t k, int64_t N, int64_t K, const void* x,
                          rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* stream);

/*
 * rb_gemv_variant -- rb_gemv for two cheap weight variants:
 *   zero_one = 1: the plane bits are {0, 1} instead of {-1, +1}, W_hat = sum_i g_i (.) B01_i (.) h_i
 *     [SigmoidBitLinear blog: a weight binarizes to {0, scale_row}: a set bit keeps the row's
 *     scale, a clear bit gives 0], so y = sum_i g_i (.) T_i with T_i the masked sum of h_i (.) x
 *     over the set bits (the +-1 product's 2 T - S without the 2 and the S);
 *   mu (optional, [N] in scale_dtype): a per-row offset, W_hat += mu 1^T, y += mu (.) sum_k x
 *     [BTC 2.1.1: zero-mean preprocessing shifts each row by its mean before binarizing].
 *   zero_one = 0 and mu = NULL is rb_gemv. mu requires h = NULL (else RB_ERR_UNSUPPORTED); zero_one
 *   must be 0 or 1. Other arguments, limits, workspace and errors as rb_gemv.
 */
rb_status rb_gemv_variant(const uint32_t* planes, int64_t ldp, const void* g, const void* h, const void* mu,
                          int32_t zero_one, rb_dtype scale_dtype, int32_t k, int64_t N, int64_t K, const void* x,
                          rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * rb_gemm_small -- the same product for larger batches, on the matrix cores: the bits
 *   of each plane are expanded to +-h_i fp16 tiles and multiplied with the fp16
 *   activations (fp32 accumulation); y = sum_i g_i (.) acc_i.
 *   Arguments as rb_gemv, except: x_dtype must be RB_F16; 1 <= M <= 4096; K must be a
 *   multiple of 64 and at most 2^22, ldp even and at most 2^20; a non-NULL h must be RB_F16 (scale_dtype
 *   RB_F16, else RB_ERR_UNSUPPORTED) and 16-byte aligned. Rows of y past M and columns
 *   past N are not written. When the row and batch tiles are too few to fill the GPU (e.g.
 *   N = 4096), K is split across blocks and the partial sums meet in the workspace:
 *   rb_workspace_bytes(RB_OP_GEMM_SMALL, k, N, K, M) bytes (the zero region, then fp32
 *   [chunks][M][N]; 0 when no split is used), 4-byte aligned; the partials are scratch. The chunks are added in a fixed
 *   order, so the result is deterministic.
 *   With fp16 g and h = NULL, +-g_i itself is the expanded operand and all planes share
 *   one accumulator; otherwise each plane's sum is scaled by g_i in fp32.
 */
rb_status rb_gemm_small(const uint32_t* planes, int64_t ldp, const void* g, const void* h,
                        rb_dtype scale_dtype, int32_t k, int64_t N, int64_t K, const void* x,
                        rb_dtype x_dtype, int64_t M, void* y, rb_dtype y_dtype, void* ws,
                        size_t ws_bytes, void* stream);

/*
 * rb_codebook_encode -- nearest binary codeword of every v-column block of a sign plane.
 *   [BTC 2.1.1: the sign matrix is cut into v-dimensional +-1 sub-vectors, each stored
 *   as the index of a codeword; distance is Hamming, via XOR + popcount]
 *     block j of row n = columns v*j .. v*j+v-1 of the plane (bit t = column v*j+t;
 *     columns >= K count as +1, i.e. bit 1); idx[n][j] = argmin_c popcount(block ^ C[c]),
 *     ties to the lowest c.
 *
 *   sign_plane  [N][ldp] uint32 in the plane format above (one plane), 16-byte aligned
 *   codebook    [c] uint32, codeword in the low v bits (upper bits must be 0)
 *   c           1..65536 (index width ceil(log2 c) <= 16 bits, [BTC 5.2])
 *   v           1..32
 *   idx         output [N][ceil(K/v)] uint16
 */
rb_status rb_codebook_encode(const uint32_t* sign_plane, int64_t ldp, int64_t N, int64_t K,
                             const uint32_t* codebook, int32_t c, int32_t v, uint16_t* idx,
                             void* stream);

/*
 * rb_codebook_encode_table -- rb_codebook_encode through a table of the nearest codeword of
 *   every one of the 2^v possible blocks, built first by a breadth-first search over the
 *   hypercube from all codewords at once (layer d + 1 takes the lowest index among the
 *   distance-d neighbours, which is the lowest index among the nearest codewords). The result is
 *   identical to rb_codebook_encode's, bit for bit; the work is about 2^v x (a few layers) table
 *   visits plus one lookup per block instead of N ceil(K/v) c distance evaluations.
 *   v 1..24 and N ceil(K/v) below 2^32 (else RB_ERR_UNSUPPORTED); codewords must hold only
 *   their low v bits (the table is
 *   indexed by them); ws rb_codebook_table_bytes(v) bytes (4 << v, plus 128), 4-byte aligned,
 *   scratch (no zero-filling needed). Other arguments as rb_codebook_encode.
 */
size_t rb_codebook_table_bytes(int32_t v);
rb_status rb_codebook_encode_table(const uint32_t* sign_plane, int64_t ldp, int64_t N, int64_t K,
                                   const uint32_t* codebook, int32_t c, int32_t v, uint16_t* idx, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * Binary codebook learning (binary K-means over the v-column sign blocks of one plane).
 *   [BTC 2.1.1: E-step = nearest codeword in Hamming distance (rb_codebook_encode); M-step =
 *   each codeword becomes the sign of the sum of its members' +-1 vectors, zeros -> +1; when
 *   the number M of distinct blocks is below the codebook size c, the size becomes M]
 * Blocks are cut as in rb_codebook_encode (columns >= K count as +1). Everything is integer:
 * results are exact and deterministic.
 *
 * rb_codebook_learn_workspace_bytes -- workspace of the three calls below for an N x K plane
 *   and c codewords of v bits (blocks = N ceil(K/v)); the largest of:
 *   - the M-step's records, a uint32 pattern and a byte of index per block (the blocks sorted
 *     by the high byte of their codeword index), 256 counts per 8192 blocks and 256 bucket
 *     totals (together rounded up to 64 words), then 256 (v + 1) counts per slice of at most
 *     4096 blocks, for floor(blocks / 4096) + min(ceil(c / 256), blocks) slices;
 *   - the per-codeword counters of the learning loop (c (v + 1) uint32);
 *   - rb_codebook_distinct's 2^v-byte pattern map (rounded up to 16 bytes) and 2^v-bit bitmap;
 *   - when rb_codebook_learn encodes through the nearest-codeword table (v <= 24 and
 *     N ceil(K/v) c > 64 x 2^v, where the table is the cheaper search), that table.
 *   0 for invalid sizes. N ceil(K/v) must be below 2^32 (else RB_ERR_UNSUPPORTED).
 */
size_t rb_codebook_learn_workspace_bytes(int64_t N, int64_t K, int32_t c, int32_t v);

/* rb_codebook_mstep -- one M-step: codeword j = majority vote, bit by bit, of the blocks with
 *   idx == j (a tie gives 1, i.e. +1); a codeword no block chose keeps its value.
 *   sign_plane [N][ldp] as in rb_codebook_encode;  v 1..32;  c 1..65536
 *   idx        [N][ceil(K/v)] uint16, each < c (an entry >= c is skipped)
 *   codebook   [c] uint32, read and updated in place (low v bits)
 *   counts     optional output [c] uint32: blocks per codeword (NULL: not written)
 *   ws         rb_codebook_learn_workspace_bytes(N, K, c, v) bytes, 4-byte aligned */
rb_status rb_codebook_mstep(const uint32_t* sign_plane, int64_t ldp, int64_t N, int64_t K, int32_t v,
                            const uint16_t* idx, uint32_t* codebook, int32_t c, uint32_t* counts, void* ws,
                            size_t ws_bytes, void* stream);

/* rb_codebook_distinct -- M = the number of distinct blocks, written to *n_distinct (device
 *   int32). If M < c the codebook becomes the distinct blocks in ascending order, entries M..c-1
 *   repeating the largest (a repeat never wins a tie, so the effective size is M); otherwise the
 *   codebook is not touched. v 1..24 (a flag byte and a bit per each of the 2^v patterns live in
 *   ws). */
rb_status rb_codebook_distinct(const uint32_t* sign_plane, int64_t ldp, int64_t N, int64_t K, int32_t v,
                               uint32_t* codebook, int32_t c, int32_t* n_distinct, void* ws, size_t ws_bytes,
                               void* stream);

/* rb_codebook_learn -- rb_codebook_distinct, then `iters` iterations (0..1000) of E-step
 *   (rb_codebook_encode) and M-step (rb_codebook_mstep), then a final E-step: codebook holds
 *   the caller's initial codebook on entry and the learned one on return, idx (output
 *   [N][ceil(K/v)] uint16) the nearest codeword of every block. v 1..24. */
rb_status rb_codebook_learn(const uint32_t* sign_plane, int64_t ldp, int64_t N, int64_t K, int32_t v,
                            uint32_t* codebook, int32_t c, int32_t iters, uint16_t* idx, int32_t* n_distinct,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * rb_codebook_gemv -- product with codebook-compressed signs and group scales.
 *   [BTC 2.1.2 (LUT-GEMM: sums of input blocks against codeword patterns are precomputed
 *   and accumulated by weight index, with no dequantisation) and 3.2.1 (one scale per
 *   16 weights)]
 *     y[m][n] = sum_c s[n][c/group] * (+-1 bit (c mod v) of C[idx[n][c/v]]) * x[m][c]
 *
 *   idx       [N][ceil(K/v)] uint16 (each < c)
 *   codebook  [c] uint32 as for rb_codebook_encode
 *   s         [N][ceil(K/group)] fp16 group scales
 *   group     a power of two in 2..64
 *   x         [M][K] fp16, 16-byte aligned;  M = 1..4
 *   y         output [M][N] fp16
 *   ws        rb_workspace_bytes(RB_OP_CODEBOOK_GEMV, 1, N, K, M) bytes (may be 0)
 */
rb_status rb_codebook_gemv(const uint16_t* idx, const uint32_t* codebook, int32_t c, int32_t v,
                           const void* s, int32_t group, int64_t N, int64_t K, const void* x,
                           int64_t M, void* y, void* ws, size_t ws_bytes, void* stream);

/*
 * rb_svid_init -- function-aware initialization of k residual paths (deploy-time, before
 * training or packing).
 *   [RaBiT, "Method step details", Algorithm 1: I/O channel importance scaling, then
 *   iterative residual SVID over T_max = 20 Gauss-Seidel sweeps with rank-1 SVD scales,
 *   then the scales mapped back to the original domain]
 *     W' = s_out^a_out (.) W (.) s_in^a_in; paths start at 0; T sweeps, in each path
 *     i = 0..k-1 in turn: R_i = W' - sum_{j != i} g'_j (.) B_j (.) h'_j (the other paths at
 *     their latest values), B_i = sign(R_i) (0 -> +1), (g'_i, h'_i) = (sqrt(s) u, sqrt(s) v)
 *     for the top singular triple (s, u, v) of |R_i|; g_i = g'_i / s_out^a_out,
 *     h_i = h'_i / s_in^a_in.
 *   The singular pair is found by P power iterations (alternating |R| v and |R|^T u passes,
 *   warm-started from the previous sweep), in fp32, deterministic.
 *
 *   W        [N][ldw] fp32 (w_dtype must be RB_F32), 16-byte aligned, ldw >= K a multiple of 4
 *   k        1..4 paths;  T  sweeps, 1..1000;  P  power iterations per path update, 1..64
 *   s_in     [K] fp32 input-column importance, > 0, or NULL (all ones);  a_in its exponent
 *   s_out    [N] fp32 output-row importance, > 0, or NULL (all ones);  a_out its exponent
 *   planes   output [k][N][ldp] uint32 sign planes (plane format above, padding bits 0), 16-byte
 *            aligned, ldp >= ceil(K/32); words past ceil(K/32) are not written
 *   g        output [k][N] fp32 row scales;  h  output [k][K] fp32 column scales (both >= 0)
 *   ws       rb_workspace_bytes(RB_OP_SVID_INIT, k, N, K, 1) bytes, 16-byte aligned; no
 *            zero-filling needed (every call writes the scratch it reads, after the zero region)
 *   The caller owns every buffer; the call only enqueues on `stream`.
 */
rb_status rb_svid_init(const void* W, rb_dtype w_dtype, int64_t N, int64_t K, int64_t ldw, int32_t k,
                       int32_t T, int32_t P, const float* s_in, const float* s_out, float a_in, float a_out,
                       uint32_t* planes, int64_t ldp, float* g, float* h, void* ws, size_t ws_bytes,
                       void* stream);

/* ---------------------------------------------------------------------------------------
 * Coupled training of one layer: the paths are derived from one shared full-precision weight
 * on every forward; the backward is straight-through with scale gradients.
 *   [RaBiT, "Method step details", Algorithm 2]
 *     forward:  R_0 = W; for i = 1..k: B_i = sign(R_{i-1}) (0 -> +1),
 *               What_i = g_i (.) B_i (.) h_i, R_i = R_{i-1} - What_i; What = sum_i What_i and
 *               Y = X What^T.
 *     backward: dW = dY^T X (the shared weight's gradient; the derivation itself is not
 *               differentiated), dX = dY What, and with the B_i held constant
 *               dg_i[n] = sum_c dW[n,c] B_i[n,c] h_i[c], dh_i[c] = sum_n dW[n,c] B_i[n,c] g_i[n].
 *   The residual and the sum What are evaluated in fp64 in the order above (so the signs are
 *   those of an fp64 evaluation); What is rounded once to the activation type. The dense
 *   products run on the matrix cores through rocBLAS (fp16/bf16 operands, fp32 accumulation)
 *   on one rocBLAS handle per device, created on the first call on that device; rocBLAS keeps
 *   its own device workspace with the handle. These are the only entry points that allocate
 *   (once per device, on first use) and they serialise their rocBLAS calls on a lock.
 * Shapes and types shared by the three calls
 *   W        [N][ldw] fp32 shared weight, ldw >= K; W must be finite
 *   g, h     [k][N], [k][K] fp32 learnable scales;  k = 1..4;  1 <= N, K <= 2^28
 *   a_dtype  RB_F16 or RB_BF16: the type of X, dY, What and the GEMM operands
 *   X        [M][ldx] activations (ldx >= K);  dY [M][lddy] gradient of Y (lddy >= N);
 *            1 <= M <= 2^31 - 1; every leading dimension <= 2^31 - 1
 *   planes   [k][N][ldp] uint32 sign planes (plane format above), ldp >= ceil(K/32)
 *   What     [N][ldwh] effective weight in a_dtype, ldwh >= K
 *   All 4-byte (fp32, planes) and 2-byte (fp16/bf16) buffers must be aligned to their element
 *   size; fp32 and fp16/bf16 outputs must not overlap any input.
 * --------------------------------------------------------------------------------------- */

/* rb_qat_derive -- the forward derivation alone: planes (padding bits 0; words past
 * ceil(K/32) not written) and What (columns past K not written), one pass over W. */
rb_status rb_qat_derive(const float* W, int64_t N, int64_t K, int64_t ldw, int32_t k, const float* g,
                        const float* h, uint32_t* planes, int64_t ldp, void* What, rb_dtype a_dtype,
                        int64_t ldwh, void* stream);

/* rb_qat_forward -- rb_qat_derive, then Y [M][ldy] = X What^T (ldy >= N) with y_dtype RB_F32
 * or a_dtype. Planes and What are outputs kept for the backward. The product runs on rocBLAS,
 * or on the library's matrix-core kernel (rb_qat_matmul, RB_QAT_ENGINE_MFMA) for a shape where
 * rb_qat_autotune timed that kernel at least as fast. */
rb_status rb_qat_forward(const float* W, int64_t N, int64_t K, int64_t ldw, int32_t k, const float* g,
                         const float* h, const void* X, rb_dtype a_dtype, int64_t M, int64_t ldx,
                         uint32_t* planes, int64_t ldp, void* What, int64_t ldwh, void* Y, rb_dtype y_dtype,
                         int64_t ldy, void* stream);

/* rb_qat_matmul -- the forward's product alone, on a chosen engine.
 *   [RaBiT "Method step details", Algorithm 2: the layer multiplies by the effective weight]
 *   Y [M][ldy] = X What^T, X [M][ldx] and What [N][ldwh] in a_dtype (RB_F16 or RB_BF16), fp32
 *   accumulation of the exact products, Y in RB_F32 or a_dtype (rounded to nearest even).
 *   Rows of Y are M, columns N; elements past N in a row are not written.
 *   engine  RB_QAT_ENGINE_AUTO: as rb_qat_forward chooses; RB_QAT_ENGINE_MFMA: the library's
 *           matrix-core kernel (v_mfma_f32_32x32x16, 8 waves per 128 x 256 output tile), which needs
 *           X and What 16-byte aligned, ldx and ldwh multiples of 8, K a multiple of 32, and
 *           M*ldx and N*ldwh below 2^30 elements (else RB_ERR_UNSUPPORTED); RB_QAT_ENGINE_ROCBLAS: rocBLAS
 *           (the autotuned kernel if rb_qat_autotune chose one). The engines sum in different
 *           orders, so their results may differ in the last fp32 bits. */
typedef enum rb_qat_engine { RB_QAT_ENGINE_AUTO = 0, RB_QAT_ENGINE_MFMA = 1, RB_QAT_ENGINE_ROCBLAS = 2 } rb_qat_engine;
rb_status rb_qat_matmul(const void* X, rb_dtype a_dtype, int64_t M, int64_t ldx, const void* What, int64_t ldwh,
                        int64_t N, int64_t K, void* Y, rb_dtype y_dtype, int64_t ldy, int32_t engine, void* stream);

/* rb_qat_backward -- from the forward's X, What and planes and the incoming dY:
 *   dW   output [N][lddw] fp32 (lddw >= K), the shared weight's gradient
 *   dX   output [M][lddx] (lddx >= K), dx_dtype RB_F32 or a_dtype
 *   dg   output [k][N] fp32;  dh  output [k][K] fp32 (fixed-order fp32 sums: deterministic for
 *        a given dW)
 *   ws   rb_workspace_bytes(RB_OP_QAT_BACKWARD, k, N, K, M) bytes, 16-byte aligned, for the
 *        partial sums of dg and dh; no zero-filling needed. */
rb_status rb_qat_backward(const void* dY, rb_dtype a_dtype, int64_t M, int64_t lddy, const void* X, int64_t ldx,
                          const void* What, int64_t ldwh, const uint32_t* planes, int64_t ldp, const float* g,
                          const float* h, int32_t k, int64_t N, int64_t K, float* dW, int64_t lddw, void* dX,
                          rb_dtype dx_dtype, int64_t lddx, float* dg, float* dh, void* ws, size_t ws_bytes,
                          void* stream);

/* rb_qat_autotune -- choose the GEMM kernels of the training layer for one shape: for each of
 * the three products of rb_qat_forward / rb_qat_backward with these sizes, leading dimensions
 * and types, times rocBLAS's default and every kernel rocBLAS lists for the problem on the
 * caller's buffers (for the forward product, the library's matrix-core kernel as well, where
 * it applies), and records the fastest for this device (process-wide; later calls with the
 * same shape use it). A setup call: it runs a few thousand products and synchronises
 * `stream` before returning. X, dY and What are read; Y, dW and dX are overwritten with
 * unspecified values. Arguments as in rb_qat_forward / rb_qat_backward. Different kernels
 * may round differently (all accumulate in fp32). */
rb_status rb_qat_autotune(const void* X, const void* dY, rb_dtype a_dtype, int64_t M, int64_t ldx, int64_t lddy,
                          const void* What, int64_t ldwh, int64_t N, int64_t K, void* Y, rb_dtype y_dtype,
                          int64_t ldy, float* dW, int64_t lddw, void* dX, rb_dtype dx_dtype, int64_t lddx,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RB_H_ */
