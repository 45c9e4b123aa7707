/*
 * msq.h -- block-wise mixed-precision weight-only quantized matmul, C ABI.
 *
 * What the library computes
 * -------------------------
 * A bf16 weight matrix W [N out][K in] is reordered in both directions
 * (rows by perm_row, columns by perm_col), cut into blocks of 64 rows x 128
 * columns, and every block is round-to-nearest quantized at its own bitwidth
 * b in {0,1,2,3,4,8}: asymmetric, one group of 128 along K per row per block,
 * so each (row, block) has one scale and one integer zero point; or kept at
 * b == 16, a bf16 passthrough ("TileQuant" abstract, fugumt.com page: tiles
 * kept at 16 bits beside 8-bit ones).  The codes
 * are packed into one compact buffer, segment by segment in ascending
 * bitwidth, located through a prefix-summed block-offset table.  Inference
 * then computes y = x . W^T by dequantizing every block on the fly.
 *
 *   - Precision chosen per 64x128 block after reordering rows and columns so
 *     that sensitive weights cluster into block-aligned regions:
 *     "ScaleBITS" summary page (atlas.scime.ai), section Approach; the
 *     abstract on the paper-with-me page calls this hardware-aligned,
 *     block-wise partitioning.
 *   - Scalar quantizer is RTN with group size 128: same summary page,
 *     section Limitations ("RTN-g128" is also the uniform baseline in
 *     section Key results).  Minimum precision 0 or 1 bit: section
 *     Surprising findings.
 *   - Row/column reordering costs a small activation reordering at inference:
 *     "SFMP" abstract (aiqbench page).  This library gathers x through
 *     perm_col inside its kernels and scatters y back through perm_row.
 *   - A precision map guides reconstruction into compact weight buffers that
 *     the kernel reuses: "TileQuant" abstract (fugumt page).
 *
 * Readings where the pages are silent (each is a choice of this library):
 *   - Block orientation: 64 rows along N (outputs) x 128 columns along K, so a
 *     block row holds exactly one 128-wide quantization group.
 *   - Quantizer, all in IEEE fp32 rounded after every operation:
 *       lo = min(0, min over group of w),  hi = max(0, max over group of w)
 *       qmax = 2^b - 1,  s = (hi - lo) / qmax
 *       if s == 0:  z = 0 and every code is 0
 *       else:       z = clamp(rint(-lo / s), 0, qmax)
 *                   q = clamp(rint(w / s) + z, 0, qmax)
 *     rint is round-half-to-even.  The dequantized weight is s * (q - z).
 *     b == 0 means the block is pruned: no codes, s = 0, z = 0, W-hat = 0.
 *   - Permutations use the gather convention: reordered row i is original row
 *     perm_row[i]; reordered column j is original column perm_col[j].
 *   - y comes back in the ORIGINAL row order, in fp32.
 *
 * Packed format, version 2 (MSQ_FORMAT_VERSION): version 1 plus b == 16
 * ---------------------------------------------
 * Block (r, c) covers reordered rows 64r..64r+63 and reordered columns
 * 128c..128c+127.  For element (ib, jb) of the block (0 <= ib < 64,
 * 0 <= jb < 128) define
 *     rt = ib >> 4,  n = ib & 15,  kt = jb >> 5,  kg = (jb >> 3) & 3,
 *     e = jb & 7,  lane l = n + 16*kg,  fragment F = 4*rt + kt,
 *     word d = e >> 1,  half h = e & 1.
 * For b in {1,2,4,8}: phi = 16 / b fragments share one 1 KiB chunk;
 * chunk t = F / phi, slot s = F % phi.  The b-bit code sits at bit
 * 16*h + b*s of the little-endian uint32 at byte 1024*t + 16*l + 4*d of the
 * block.  A b-bit block therefore occupies 1024*b bytes.
 * For b == 16 (phi = 1, chunk t = F) the same rule places the bf16 bit
 * pattern of the reordered weight: chunk F holds, at lane l, the eight bf16
 * values of fragment F, ready as the matrix instruction's B operand; such a
 * block occupies 16384 bytes and stores s = 0, z = 0 (the quantized kernels
 * treat it as pruned; one more pass adds its exact bf16 product).
 * For b == 3 the code q = q_lo + 4*q_hi is split into planes: q_lo (2 bits)
 * follows the b == 2 rule in chunks 0..1 and q_hi (1 bit) follows the
 * b == 1 rule in chunk 2; the block occupies 3072 bytes.
 * Every chunk is one contiguous KiB that a 64-lane wavefront fetches with
 * one 16-byte load per lane; for each slot, masking the four words of a lane
 * yields the 8 codes of one 16x32 operand fragment of a gfx950 bf16 matrix
 * instruction (row 16*rt + n, columns 32*kt + 8*kg .. +7).
 *
 * Buffer: block (r, c) starts at byte 1024 * block_offset[r][c] of codes.
 * Blocks are laid out segment by segment for b = 1, 2, 3, 4, 8, 16; inside a
 * segment in row-major (r, c) order; block_offset is the exclusive prefix
 * sum of bits over that order, in KiB.  0-bit blocks own no bytes and have
 * block_offset == MSQ_NO_BLOCK.  code_bytes = 1024 * sum(bits).
 * scale is float32 [N/64][K/128][64] and zero is uint8 [N/64][K/128][64],
 * both indexed by (block row, block column, row inside the block) in
 * reordered row order.
 *
 * Conventions
 * -----------
 *   - Pointers are device pointers unless the name ends in _host.
 *   - The caller allocates and owns every buffer; the library allocates no
 *     memory, keeps no device state and never synchronizes.  Device calls
 *     are asynchronous on the given stream.  Two stated exceptions:
 *     msq_allocate_bits reads a status back after each iteration, and
 *     msq_gemm_noalloc keeps its workspace in a static device array.
 *   - Errors are return codes.  All argument checks run before any launch,
 *     so outputs are untouched when a call returns an error.  A failed
 *     launch returns MSQ_ERR_HIP.
 *   - msq_plan validates bits and permutations on the host; the device
 *     calls trust a weight descriptor whose bits and permutations passed
 *     msq_plan.  Non-finite W or |W| >= 2^127 gives unspecified codes.
 */
#ifndef MSQ_H_
#define MSQ_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSQ_FORMAT_VERSION 2
#define MSQ_BLOCK_ROWS 64
#define MSQ_BLOCK_COLS 128
#define MSQ_NO_BLOCK 0xFFFFFFFFu
/* Largest M the decode (GEMV) kernel accepts. */
#define MSQ_GEMV_MAX_M 64
/* Largest M for which MSQ_KERNEL_AUTO picks the GEMV kernel; above it the
 * GEMM (which splits K when its tiles cannot fill the GPU) is faster. */
#define MSQ_AUTO_GEMV_MAX_M 32

typedef enum {
  MSQ_OK = 0,
  MSQ_ERR_INVALID_ARG = 1,      /* null pointer, misaligned pointer, bad enum */
  MSQ_ERR_SHAPE = 2,            /* N or K not a positive multiple of 64 / 128, M < 0 */
  MSQ_ERR_BITS = 3,             /* a bits entry outside {0,1,2,3,4,8,16} */
  MSQ_ERR_PERM = 4,             /* perm_row or perm_col is not a permutation */
  MSQ_ERR_BUFFER_TOO_SMALL = 5, /* code_bytes or workspace smaller than needed */
  MSQ_ERR_HIP = 6,              /* a HIP launch or runtime call failed */
  MSQ_ERR_UNSUPPORTED = 7       /* e.g. forcing the GEMV kernel with M > 64 */
} msq_status;

typedef enum {
  MSQ_KERNEL_AUTO = 0,  /* GEMV for M <= MSQ_AUTO_GEMV_MAX_M, GEMM otherwise */
  MSQ_KERNEL_GEMV = 1,  /* decode kernel; M <= MSQ_GEMV_MAX_M */
  MSQ_KERNEL_GEMM = 2   /* prefill kernel; any M >= 1 */
} msq_kernel;

/* Buffer sizes for one weight matrix, filled by msq_plan. */
typedef struct {
  int64_t code_bytes;          /* 1024 * sum(bits) */
  int64_t scale_bytes;         /* 4 * N * K / 128 */
  int64_t zero_bytes;          /* N * K / 128 */
  int64_t offset_bytes;        /* 4 * (N/64) * (K/128) */
  int64_t blocks_per_bits[17]; /* histogram of bits; index = bitwidth */
  double mean_bits;            /* sum(bits) / number of blocks */
} msq_sizes;

/* Descriptor of one packed weight matrix.  Caller-owned; the library reads
 * the pointers and never frees them. */
typedef struct {
  int64_t N, K;               /* N % 64 == 0, K % 128 == 0, both > 0 */
  const uint8_t *bits;        /* [N/64][K/128], values in {0,1,2,3,4,8,16} */
  const int32_t *perm_row;    /* [N]: reordered row i <- original row perm_row[i] */
  const int32_t *perm_col;    /* [K]: reordered col j <- original col perm_col[j]; 16-byte aligned */
  uint32_t *block_offset;     /* [N/64][K/128] in KiB; MSQ_NO_BLOCK for 0-bit */
  uint8_t *codes;             /* [code_bytes], 256-byte aligned */
  float *scale;               /* [N/64][K/128][64], 16-byte aligned */
  uint8_t *zero;              /* [N/64][K/128][64], 16-byte aligned */
  int64_t code_bytes;         /* size of the codes buffer in bytes */
  int64_t tile16_blocks;      /* number of 16-bit blocks (blocks_per_bits[16] of msq_plan);
                                 trusted: msq_gemm skips the 16-bit pass when it is 0 */
} msq_weight;

/* Host only; needs no GPU.  Validates N, K, the bit map and both
 * permutations (host copies) and fills *out with the buffer sizes.
 * Block-wise precision map and reordering: "ScaleBITS" summary page,
 * section Approach.  Returns MSQ_ERR_SHAPE, MSQ_ERR_BITS, MSQ_ERR_PERM or
 * MSQ_ERR_INVALID_ARG (null pointer); *out is untouched on error. */
msq_status msq_plan(int64_t N, int64_t K, const uint8_t *bits_host,
                    const int32_t *perm_row_host, const int32_t *perm_col_host,
                    msq_sizes *out);

/* Quantizes and packs W (bf16 bit patterns, [N][K] row-major, original
 * order, 16-byte aligned) into w->block_offset, w->codes, w->scale and
 * w->zero, asynchronously on stream (no host synchronization).  RTN-g128 per
 * block at the block's bitwidth ("ScaleBITS" summary page, sections Approach
 * and Limitations); compact per-bitwidth buffers ("TileQuant" abstract).
 * Results are bit-exact against the quantizer and format stated at the top
 * of this header.  Like every device call it trusts the descriptor: w->bits,
 * w->perm_row and w->perm_col must be what msq_plan accepted, w->code_bytes
 * at least msq_plan's code_bytes and w->tile16_blocks its
 * blocks_per_bits[16].  The kernels never read outside W or the permutations
 * and never write outside the buffers the descriptor sizes, even for a bad
 * descriptor (indices are clamped, blocks past code_bytes are skipped), but
 * the results are then unspecified.  Errors: MSQ_ERR_INVALID_ARG (null or
 * misaligned pointer, negative tile16_blocks), MSQ_ERR_SHAPE, MSQ_ERR_HIP. */
msq_status msq_quantize_pack(const uint16_t *W_bf16, const msq_weight *w,
                             hipStream_t stream);

/* Bytes of device workspace msq_gemm / msq_gemm_ex need for this shape
 * (any kernel choice).  Zero for M == 0. */
size_t msq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* y = x . W^T with W dequantized block by block from the packed buffers.
 * x: bf16 bit patterns [M][K] row-major in ORIGINAL column order (16-byte
 * aligned); y: fp32 [M][N] row-major in ORIGINAL row order, fully
 * overwritten.  The activation gather through perm_col is the reordering
 * overhead of the "SFMP" abstract; the row scatter through perm_row restores
 * the original output order.  M == 0 is a no-op.  workspace must hold
 * msq_gemm_workspace_bytes(M, N, K) bytes (256-byte aligned); calls that
 * share a workspace must be ordered on one stream.  Errors:
 * MSQ_ERR_INVALID_ARG, MSQ_ERR_SHAPE, MSQ_ERR_BUFFER_TOO_SMALL, MSQ_ERR_HIP. */
msq_status msq_gemm(const uint16_t *x_bf16, int64_t M, const msq_weight *w,
                    float *y, void *workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Launch choices for msq_gemm_ex and msq_gemm_group_ex (testing and
 * benchmarking).  A zeroed struct, or a NULL pointer, gives exactly the
 * automatic choices of msq_gemm and msq_gemm_group; results never depend on
 * these fields beyond fp32 summation order.  The library reads no
 * environment variables. */
typedef struct {
  int32_t kernel;      /* msq_kernel: MSQ_KERNEL_AUTO (0), MSQ_KERNEL_GEMV or MSQ_KERNEL_GEMM */
  int32_t gemv_split;  /* decode kernel: K ranges per block row; 0 = automatic, else >= 1
                          (capped at K / 128; ranges hold at most 64 block columns) */
  int32_t gemv_waves;  /* decode kernel at M == 1: wavefronts per workgroup; 0 = automatic,
                          else 4, 8 or 16 */
  int32_t m1_prep;     /* decode kernel at M == 1: nonzero = reorder x in the separate
                          activation-prep launch even where the workgroups could do it */
  int32_t gemm_split;  /* prefill kernel: K ranges; 0 = automatic, else >= 1 (capped at
                          K / 1024) */
} msq_options;

/* Workspace bytes of msq_gemm_ex with these options (NULL = automatic, the
 * same as msq_gemm_workspace_bytes).  Zero for M <= 0, a bad shape or bad
 * options. */
size_t msq_gemm_workspace_bytes_ex(int64_t M, int64_t N, int64_t K, const msq_options *opt);

/* As msq_gemm, with the launch choices of *opt (NULL = automatic).  The
 * workspace must hold msq_gemm_workspace_bytes_ex(M, N, K, opt) bytes.
 * MSQ_ERR_UNSUPPORTED for MSQ_KERNEL_GEMV with M > 64; MSQ_ERR_INVALID_ARG
 * for an unknown kernel value, a negative split or a wavefront count other
 * than 0, 4, 8, 16. */
msq_status msq_gemm_ex(const uint16_t *x_bf16, int64_t M, const msq_weight *w,
                       float *y, void *workspace, size_t workspace_bytes,
                       const msq_options *opt, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): msq_gemm
 * with the automatic launch choices, its workspace taken from a static
 * device array of MSQ_NOALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends.  No allocation, no memset and no
 * host synchronization happen in the call; the caller still passes x and y.
 * The first call on a device looks up that device's array (the device must
 * be current, as for every call).  All calls on one GPU share its array:
 * calls that may overlap on one GPU (different streams, or threads without
 * ordering) race and give undefined results; order them on one stream.  The
 * kernels clear what they need cleared each call, so consecutive calls of
 * any shapes are independent.  Returns MSQ_ERR_BUFFER_TOO_SMALL when
 * msq_gemm_workspace_bytes(M, N, K) for the automatic kernel exceeds the
 * array (decode up to M = 64 fits every Llama-3-70B linear; prefill fits
 * while M * K * 2 plus the K-split partials stay below it), MSQ_ERR_HIP if
 * the array cannot be located, otherwise as msq_gemm. */
#define MSQ_NOALLOC_SCRATCH_BYTES (64u << 20)
msq_status msq_gemm_noalloc(const uint16_t *x_bf16, int64_t M, const msq_weight *w, float *y,
                            hipStream_t stream);

/* Most matrices one msq_gemm_group call takes. */
#define MSQ_GROUP_MAX 8

/* Bytes of device workspace msq_gemm_group needs for these count matrices
 * at M rows: about the sum of the single-call workspaces (all matrices are
 * in flight together).  Zero for M <= 0, count outside 1 .. MSQ_GROUP_MAX
 * or a bad shape. */
size_t msq_gemm_group_workspace_bytes(int64_t M, const msq_weight *const *w, int count);

/* y[i] = x[i] . W_i^T for count matrices (1 .. MSQ_GROUP_MAX), each as
 * msq_gemm computes it (at M <= MSQ_AUTO_GEMV_MAX_M the K split that fills
 * the GPU is chosen for the whole group, so results can differ from single
 * calls in fp32 summation order; with msq_options.gemv_split set they are
 * the same bit for bit).  For the decode step of a layer, whose q, k, v
 * projections (and gate, up) read the same activation: at M == 1 one
 * decode launch covers all matrices, their workgroups running side by side
 * (matrices whose K is split into several ranges add one activation-prep
 * launch for all of them; the others reorder x inside their workgroups) ("TileQuant" abstract: local accumulation
 * to reduce memory traffic; the grouping itself is this library's).  At
 * M in 2 .. MSQ_AUTO_GEMV_MAX_M: one activation-gather launch and one
 * decode launch cover all matrices (matrices with several K ranges add
 * them up in the decode launch's last arriving workgroups).  At M > MSQ_AUTO_GEMV_MAX_M, when the matrices' tiles
 * fill the GPU (prefill), one activation-gather launch and one GEMM launch
 * cover all matrices, the tiles of the smaller ones filling the compute
 * units the larger ones leave idle; with fewer tiles the matrices are
 * computed one after the other as by msq_gemm.  Matrices with 16-bit
 * blocks add their 16-bit pass after the decode launches.  x,
 * w and y are host arrays of count device pointers / descriptors; x[i] may
 * repeat the same activation.  workspace must hold
 * msq_gemm_group_workspace_bytes(M, w, count) bytes (256-byte aligned).
 * Errors as msq_gemm; MSQ_ERR_INVALID_ARG also for a null array or count
 * outside 1 .. MSQ_GROUP_MAX. */
msq_status msq_gemm_group(const uint16_t *const *x_bf16, int64_t M,
                          const msq_weight *const *w, float *const *y, int count,
                          void *workspace, size_t workspace_bytes, hipStream_t stream);

/* msq_gemm_group_workspace_bytes and msq_gemm_group with the launch choices
 * of *opt (NULL = automatic; kernel must be MSQ_KERNEL_AUTO, since the
 * grouping follows the automatic kernel choice).  Errors as msq_gemm_group,
 * plus MSQ_ERR_INVALID_ARG for bad options. */
size_t msq_gemm_group_workspace_bytes_ex(int64_t M, const msq_weight *const *w, int count,
                                         const msq_options *opt);
msq_status msq_gemm_group_ex(const uint16_t *const *x_bf16, int64_t M,
                             const msq_weight *const *w, float *const *y, int count,
                             void *workspace, size_t workspace_bytes, const msq_options *opt,
                             hipStream_t stream);

/* ---- bitwidth allocation under a memory budget ---------------------------
 * Chooses a bitwidth per 64x128 block, from {0, 1, 2, 3, 4, 8}, so as to
 * maximise the sum of per-block utilities with the sum of the chosen bits at
 * most the budget: the knapsack over block bitwidths that the ScaleBITS
 * summary page (sections Approach and Key results) solves with a batched
 * approximation to greedy.  The pages give no batching rule; this library's
 * reading: each iteration orders every block's next one-level step by fp32
 * ratio (u[l+1] - u[l]) / (bits[l+1] - bits[l]) descending, ties by block
 * index ascending, and moves up the longest prefix of that order whose cost
 * is at most floor(R / 2) of the remaining budget R, or, when that prefix is
 * empty, the first step that fits R; it stops when no step fits.  All
 * blocks start at 0 bits.
 *
 * utility: device fp32 [n_blocks][6] (levels 0, 1, 2, 3, 4, 8 bits), finite,
 *   4-byte aligned; read only.  bits: device uint8 [n_blocks], written.
 * budget_bits: sum over blocks of the allowed bits per weight (for an average
 *   of b bits, floor(b * n_blocks)); counts codes only.
 * workspace: device, 256-byte aligned, at least msq_alloc_workspace_bytes.
 * iterations: host int32 receiving the number of batched iterations; may be
 *   NULL.
 * Blocking: the host reads a small status back after every iteration and
 *   returns when the allocation is written (stream synchronised).
 * Errors: MSQ_ERR_INVALID_ARG (null or misaligned pointer, a non-finite
 *   utility), MSQ_ERR_SHAPE (n_blocks outside [1, MSQ_ALLOC_MAX_BLOCKS] or a
 *   negative budget), MSQ_ERR_BUFFER_TOO_SMALL, MSQ_ERR_HIP. */
#define MSQ_ALLOC_MAX_BLOCKS (1 << 28)
/* Bytes of workspace for n_blocks; 0 for n_blocks outside [1,
 * MSQ_ALLOC_MAX_BLOCKS] or when hipCUB cannot size its sort and scan storage. */
size_t msq_alloc_workspace_bytes(int64_t n_blocks);
msq_status msq_allocate_bits(const float *utility, int64_t n_blocks, int64_t budget_bits,
                             uint8_t *bits, void *workspace, size_t workspace_bytes,
                             int32_t *iterations, hipStream_t stream);

/* ---- bi-directional channel reordering -----------------------------------
 * perm_row and perm_col for msq_quantize_pack from a per-weight saliency map:
 * rows and columns are ordered by their total saliency, descending, ties by
 * index ascending, so that salient weights gather in the leading block rows
 * and block columns.  The ScaleBITS summary page (section Approach) reorders
 * channels in both directions so that sensitive weights cluster into
 * block-aligned regions, and (section Limitations) leaves the Q and K
 * projections out of the row reordering: reorder_rows = 0 gives the identity
 * perm_row.  The SFMP abstract aggregates salient weights by row and column
 * reordering.  The pages give no rule; sorting by total saliency is this
 * library's reading.
 *
 * saliency: device fp32 [N][K] row-major, >= 0 and finite (not checked),
 *   16-byte aligned; N a multiple of 64 up to MSQ_REORDER_MAX_N, K a multiple
 *   of 128 up to MSQ_REORDER_MAX_K.  perm_row: device int32 [N], perm_col:
 *   device int32 [K], written (gather convention: reordered row i is
 *   original row perm_row[i]).  Row and column sums are fp32 in a fixed
 *   order, so the result is reproducible.  Asynchronous on the stream.
 * Errors: MSQ_ERR_INVALID_ARG (null or misaligned pointer), MSQ_ERR_SHAPE,
 *   MSQ_ERR_BUFFER_TOO_SMALL, MSQ_ERR_HIP. */
#define MSQ_REORDER_MAX_N (1 << 20)
#define MSQ_REORDER_MAX_K 32768
/* Bytes of workspace for an N x K map; 0 for a refused shape or when hipCUB
 * cannot size its sort storage. */
size_t msq_reorder_workspace_bytes(int64_t N, int64_t K);
msq_status msq_reorder_channels(const float *saliency, int64_t N, int64_t K, int reorder_rows,
                                int32_t *perm_row, int32_t *perm_col, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* Static English text for a status code; never NULL.  Takes an int so that
 * any value a caller holds, including one outside the enum, is defined input
 * ("unknown status"). */
const char *msq_status_string(int status);

/* MSQ_FORMAT_VERSION of the library that was loaded. */
int msq_format_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MSQ_H_ */
