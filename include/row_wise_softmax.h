/*
 * row_wise_softmax.h -- C ABI of the MI355X (gfx950) fused row-softmax library.
 *
 * The operation (every entry point that computes): for each row i of a
 * row-major matrix x with `cols` columns,
 *
 *     y[i, j] = exp(x[i, j] - m_i) / sum_k exp(x[i, k] - m_i),   m_i = max_k x[i, k]
 *
 * -- the softmax with the row max subtracted first so that large entries
 * cannot overflow ("I Wrote My First GPU Kernel", section "What Fusion
 * Actually Does"; "fused-softmax-roofline", the row-softmax fragment), fused
 * into one pass that reads each element once and writes it once (same two
 * pages), with -inf entries contributing exactly 0 and receiving exactly +0
 * ("GPU Kernels - Implementing and optimizing Softmax", section "Baseline &
 * Triton Softmax kernel").  A row whose entries are all -inf gets all +0.
 * Arithmetic is fp32 for every storage type; fp16 and bf16 outputs are rounded
 * to nearest even.  +inf and NaN inputs are outside the contract.
 *
 * Layout: row i occupies elements [i * row_stride, i * row_stride + cols) of
 * its buffer; `row_stride` counts ELEMENTS and is shared by input and output
 * (the single stride of "Kernel Fusion", section "A fused softmax in Triton").
 * Elements between `cols` and `row_stride` are never read or written.
 *
 * Ownership: the caller owns both device buffers (and any workspace).  The
 * library allocates no device memory, keeps no pointer after returning, never
 * synchronises the host and never pre-fills `out` ("I Wrote My First GPU
 * Kernel", section "The Honest Part", on the cost of zero-filling an output
 * the kernel overwrites anyway).  It writes every out[i, j < cols] once, with
 * one exception: softmax_fwd's split of few, very wide rows (below) keeps
 * partial results in the first 8 bytes of every 16 KiB tile of `out` between
 * its kernels before writing the final values there.
 *
 * Aliasing: in == out (exactly in place) is allowed; any other overlap of the
 * two extents is rejected with SOFTMAX_ERR_OVERLAP.
 *
 * Asynchrony: computing calls enqueue work on `stream` (a hipStream_t passed
 * as void*; NULL is the default stream) and return.  SOFTMAX_OK means the
 * launch was accepted; a fault during execution surfaces as a HIP error at the
 * caller's next synchronisation.  Calls are stateless and thread-safe, and
 * make no allocation or memset, so they may be captured in a hipGraph.
 *
 * Errors: every entry point returns a status and never prints, throws or
 * aborts.  Arguments are validated before any HIP call.  rows == 0 or
 * cols == 0 returns SOFTMAX_OK without launching (pointers may then be NULL).
 */
#ifndef ROW_WISE_SOFTMAX_H
#define ROW_WISE_SOFTMAX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage types (input and output share one). */
#define SOFTMAX_F32 0
#define SOFTMAX_F16 1
#define SOFTMAX_BF16 2

/* Status codes. */
#define SOFTMAX_OK 0
#define SOFTMAX_ERR_NULL_POINTER 1 /* rows * cols > 0 with a NULL buffer, or a NULL out-parameter */
#define SOFTMAX_ERR_BAD_SHAPE 2    /* negative dims, row_stride < cols, cols > 2^30, or a byte extent past INT64_MAX */
#define SOFTMAX_ERR_BAD_DTYPE 3    /* dtype not one of SOFTMAX_F32 / F16 / BF16 */
#define SOFTMAX_ERR_OVERLAP 4      /* in and out overlap without being equal */
#define SOFTMAX_ERR_BAD_KERNEL 5   /* forced kernel id unknown, of another dtype or kind, or unable to take this width / alignment */
#define SOFTMAX_ERR_HIP 6          /* the HIP runtime refused the launch */
#define SOFTMAX_ERR_BAD_SCALE 7    /* causal entry points: scale not > 0, or scale * log2(e) not below 3e38 */
#define SOFTMAX_ERR_SCRATCH_LIMIT 8 /* softmax_fwd_split_noalloc: the split needs more than its static scratch */

/* Kernel variants of the compiled table. */
#define SOFTMAX_VARIANT_PACKED 0 /* L lanes of a wave per row, 64/L rows per wave (narrow rows) */
#define SOFTMAX_VARIANT_ROW 1    /* one workgroup per row, row held in registers (single pass) */
#define SOFTMAX_VARIANT_ONLINE 2 /* one workgroup per row, two reads + one write (any width) */
#define SOFTMAX_VARIANT_ROW_PF 3 /* row kernel, persistent: each workgroup loops over rows and prefetches the next */
#define SOFTMAX_VARIANT_ROW16 4  /* 16-bit types: one workgroup per row, the row kept in registers as stored (wide rows) */

/*
 * softmax_fwd -- the fused row softmax, with the library's width dispatch.
 *   in, out     device pointers to rows x row_stride elements of `dtype`
 *               (the last row needs only `cols`), element-aligned.  Rows move
 *               in 16-byte accesses whatever the width, pitch and offset as
 *               long as in and out sit at the same offset within their
 *               16-byte chunks (two tensors of one layout from one
 *               allocator): rows that start and end on 16-byte boundaries on
 *               the aligned kernels, others on the any-alignment kernels,
 *               which read a row's chunks whole (masking the neighbouring
 *               rows' elements) and write the chunks it shares with its
 *               neighbours element by element.  In and out at different
 *               offsets take a scalar path of the same results.
 *   rows, cols  matrix shape; the softmax runs along each row.
 *   row_stride  elements between the starts of consecutive rows (>= cols).
 *   dtype       SOFTMAX_F32, SOFTMAX_F16 or SOFTMAX_BF16.
 *   stream      hipStream_t as void*.
 * The width dispatch follows the pages' advice to pick the path by measured
 * width crossovers ("fused-softmax-roofline", the closing discussion of
 * where the fused kernel loses) and to tune block shape per width rather than
 * by one formula ("GPU Kernels - Implementing and optimizing Softmax",
 * sections "CUDA scaling threads" and "Autotuning").
 * Few, very wide rows, out of place on the 16-byte path, take the split path
 * of softmax_fwd_split below without a workspace: each tile's (max, sum) pair
 * is kept in the first 8 bytes of that tile's own output.  Calls of up to
 * 1024 tiles merge the pairs in the second kernel, whose last workgroup of
 * each row writes the tiles' first accesses after the others have read them
 * (a counter in the row's first slot); larger ones run a third kernel that
 * merges each row's pairs between the other two.  One workgroup per row would
 * keep only `rows` of the 256 compute units busy.  The measured lines: fp32
 * rows of >= 2 MiB up to 192 rows, >= 1 MiB up to 128, > 256 KiB up to 64,
 * >= 224 KiB up to 32, >= 192 KiB up to 16; fp16 / bf16 rows of >= 2 MiB up to
 * 256 rows, >= 1 MiB up to 192, >= 512 KiB up to 128, >= 192 KiB up to 64,
 * >= 128 KiB up to 16.  Results are bit-identical to softmax_fwd_split's.
 */
int softmax_fwd(const void *in, void *out, int64_t rows, int64_t cols, int64_t row_stride,
                int dtype, void *stream);

/*
 * softmax_fwd_causal -- the scaled, causally masked row softmax: row i keeps
 * columns j <= i + diag, and
 *
 *     y[i, j] = exp(scale x[i, j] - M_i) / sum_{k <= i + diag} exp(scale x[i, k] - M_i)
 *
 * for kept j (M_i the max of scale x over the kept columns), y[i, j] = +0 for
 * masked j; rows with no kept column, or whose kept entries are all -inf,
 * are all +0.  This is the score scaling and causal mask applied before the
 * softmax in "Dissecting Memory Bandwidth & SRAM Tiling in Triton", section
 * "Writing the Kernel in OpenAI Triton" (scale 1/sqrt(head dim), mask
 * column > row), fused into the softmax: masked inputs are never read, so a
 * causal square reads about half of its input while still writing all of
 * its output.  diag = 0 is that mask; diag = cols - rows aligns it to the
 * bottom-right corner; any int64 value is accepted.
 *   scale  > 0 with scale * log2(e) below 3e38 (else SOFTMAX_ERR_BAD_SCALE);
 *          it is folded into the exponent as one fp32 coefficient
 *          scale * log2(e).
 * Other arguments, layout, ownership, aliasing and errors as softmax_fwd.
 */
int softmax_fwd_causal(const void *in, void *out, int64_t rows, int64_t cols, int64_t row_stride,
                       float scale, int64_t diag, int dtype, void *stream);

/*
 * softmax_fwd_causal_batched -- softmax_fwd_causal over a batch of score
 * matrices stacked row-wise, such as attention scores [batch][heads][n][m]
 * seen as (batch * heads * n) rows of m columns: row r of the call is row
 * i = r mod rows_per_matrix of its matrix, keeps the columns j <= i + diag,
 * and is scaled and normalised as in softmax_fwd_causal.  The mask is the one
 * "Dissecting Memory Bandwidth & SRAM Tiling in Triton" (section "Writing the
 * Kernel in OpenAI Triton") applies to every head's score matrix.
 *   rows_per_matrix  rows of one matrix (>= 1); rows must be a multiple of it
 *                    (else SOFTMAX_ERR_BAD_SHAPE; not checked for an empty
 *                    call).  rows_per_matrix == rows is softmax_fwd_causal.
 * Other arguments, layout, ownership, aliasing and errors as softmax_fwd_causal.
 */
int softmax_fwd_causal_batched(const void *in, void *out, int64_t rows, int64_t cols, int64_t row_stride,
                               int64_t rows_per_matrix, float scale, int64_t diag, int dtype, void *stream);

/*
 * softmax_fwd_kernel -- the same operation through one forced entry of the
 * compiled kernel table, for width sweeps and tests: the per-width search over
 * launch configurations of "GPU Kernels - Implementing and optimizing Softmax"
 * (sections "CUDA scaling threads" and "Autotuning").  Same arguments and
 * errors as softmax_fwd, plus SOFTMAX_ERR_BAD_KERNEL when `kernel_id` is out of
 * range, is compiled for another dtype, or cannot take this width, stride or
 * pointer alignment (see softmax_kernel_fits).
 */
int softmax_fwd_kernel(int kernel_id, const void *in, void *out, int64_t rows, int64_t cols,
                       int64_t row_stride, int dtype, void *stream);

/*
 * softmax_fwd_causal_kernel -- softmax_fwd_causal through one forced causal
 * table entry.  Plain entries are refused with SOFTMAX_ERR_BAD_KERNEL (and
 * softmax_fwd_kernel refuses causal ones).
 */
int softmax_fwd_causal_kernel(int kernel_id, const void *in, void *out, int64_t rows, int64_t cols,
                              int64_t row_stride, float scale, int64_t diag, int dtype, void *stream);

/*
 * softmax_select -- the kernel id softmax_fwd would launch for these
 * arguments, written to *kernel_id, or SOFTMAX_KERNEL_SPLIT when softmax_fwd
 * takes the split path (few, very wide rows): the choice of kernel shape by
 * row width from measured crossovers ("fused-softmax-roofline", the closing
 * discussion of where the fused kernel loses; "GPU Kernels - Implementing and
 * optimizing Softmax", section "Autotuning").  Validates like softmax_fwd;
 * launches nothing.
 */
#define SOFTMAX_KERNEL_SPLIT (-1)
int softmax_select(const void *in, const void *out, int64_t rows, int64_t cols, int64_t row_stride,
                   int dtype, int *kernel_id);

/*
 * softmax_fwd_variant -- the operation through a forced kernel variant and
 * size, the way the width sweep of "GPU Kernels - Implementing and
 * optimizing Softmax" (sections "CUDA scaling threads" and "Autotuning")
 * forces a block size per width:
 *   variant  SOFTMAX_VARIANT_PACKED, _ROW, _ONLINE, _ROW_PF or _ROW16 (16-bit only);
 *   block    packed: lanes per row (1, 2, 4, ..., 64); the others: threads per
 *            workgroup (64 x waves).
 * Of the compiled entries with that variant and size that take the call, it
 * runs the one on 16-byte accesses if any, then with the fewest accesses per
 * lane, then the fewest row groups in flight (softmax_fwd_kernel forces one
 * exact entry instead).  Same arguments and errors as softmax_fwd, plus
 * SOFTMAX_ERR_BAD_KERNEL when no such entry takes this width, stride or
 * alignment, or the variant is unknown.
 */
int softmax_fwd_variant(const void *in, void *out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
                        int variant, int block, void *stream);

/*
 * softmax_select_variant -- the variant and size (as softmax_fwd_variant
 * takes them) that softmax_fwd picks for a contiguous tensor of `cols`
 * columns of `dtype` on 16-byte-aligned buffers with many rows: the width
 * dispatch by measured crossovers ("fused-softmax-roofline", the closing
 * discussion of where the fused kernel loses).  Launches nothing.
 * Errors: NULL_POINTER, BAD_DTYPE, BAD_SHAPE (cols < 1 or > 2^30).
 */
int softmax_select_variant(int64_t cols, int dtype, int *variant, int *block);

/* softmax_select for softmax_fwd_causal: the causal entry it would launch. */
int softmax_select_causal(const void *in, const void *out, int64_t rows, int64_t cols, int64_t row_stride,
                          int dtype, int *kernel_id);

/* Number of entries in the compiled kernel table (ids 0 .. n-1). */
int softmax_num_kernels(void);

/*
 * softmax_kernel_info -- the parameters of table entry `kernel_id`:
 *   dtype, variant (SOFTMAX_VARIANT_*), causal (1 for an entry of the scaled,
 *   causally masked softmax, 0 for the plain one), vec_elems (elements per memory access),
 *   lanes (packed: lanes per row; row/online: threads per row),
 *   vecs_per_lane (accesses per lane per row, or per chunk for online),
 *   groups (packed: row groups per wave in flight; else 1),
 *   block (threads per workgroup; packed: the maximum), and
 *   max_cols (widest row it takes; -1 for any).
 * Any out-pointer may be NULL.  Returns SOFTMAX_ERR_BAD_KERNEL for an unknown id.
 */
int softmax_kernel_info(int kernel_id, int *dtype, int *variant, int *causal, int *vec_elems, int *lanes,
                        int *vecs_per_lane, int *groups, int *block, int64_t *max_cols);

/* Static, human-readable name of table entry `kernel_id` (NULL if unknown). */
const char *softmax_kernel_name(int kernel_id);

/* 1 if table entry `kernel_id` can run these arguments, else 0.  Launches nothing. */
int softmax_kernel_fits(int kernel_id, const void *in, const void *out, int64_t cols,
                        int64_t row_stride, int dtype);

/* Static description of a status code. */
const char *softmax_status_string(int status);

/* Static version string of the library. */
const char *softmax_version(void);

/*
 * softmax_bench_copy -- a plain device copy of `bytes` bytes with 16-byte
 * accesses (src and dst 16-byte aligned, bytes a multiple of 16, no overlap).
 * It is the achievable read-once/write-once bandwidth a finished softmax is
 * measured against ("Kernel Fusion", section "What interviewers are listening
 * for": a fused kernel running at device-copy bandwidth is done).
 * Errors: NULL_POINTER, BAD_SHAPE (negative, or not a multiple of 16, or
 * misaligned), OVERLAP, HIP.
 */
int softmax_bench_copy(const void *src, void *dst, int64_t bytes, void *stream);

/*
 * softmax_bench_stream -- the copy's two directions timed apart, with the same
 * 16-byte accesses and grid as softmax_bench_copy, so that the bench can show
 * what a read-once/write-once kernel can reach at each size:
 *   mode 0  copy src -> dst (softmax_bench_copy);
 *   mode 1  read `bytes` from src; dst must hold 4 writable bytes, where the
 *           kernel stores one word only in the unlikely case that the XOR of
 *           all the data equals a fixed value (the store keeps the loads);
 *   mode 2  write `bytes` of a fixed pattern to dst; src is unused.
 * Errors: BAD_KERNEL (other modes), NULL_POINTER, BAD_SHAPE (negative, not a
 * multiple of 16, misaligned), OVERLAP (mode 0), HIP.
 */
int softmax_bench_stream(const void *src, void *dst, int64_t bytes, int mode, void *stream);

/*
 * softmax_bench_chunk_copy -- a copy shaped like the row kernels without their
 * arithmetic: each workgroup of `waves` waves copies one contiguous chunk of
 * waves * 64 * accesses 16-byte accesses (wave w its run of 64 * accesses,
 * each lane `accesses` loads 1 KiB apart), all loads, a barrier, then all
 * stores.  Its rate per chunk size shows what the row kernels' access
 * pattern alone allows at a given row size.
 *   (waves, accesses) in {(4,2), (8,2), (4,4), (16,2), (4,8), (8,4), (4,16),
 *   (8,8), (16,4)}; bytes a multiple of the chunk.
 * Errors: BAD_KERNEL (other shapes), BAD_SHAPE, NULL_POINTER, OVERLAP, HIP.
 */
int softmax_bench_chunk_copy(const void *src, void *dst, int64_t bytes, int waves, int accesses, void *stream);

/*
 * ---- Split-row softmax: few, wide rows ----
 *
 * With one workgroup per row, a matrix of few wide rows (say 8 x 1,048,576)
 * occupies a few of the 256 compute units.  The split path cuts every row
 * into tiles, one workgroup each: a first kernel writes each tile's (max, sum)
 * pair to a workspace, a second merges a row's pairs with the online-softmax
 * rule ("Dissecting Memory Bandwidth & SRAM Tiling in Triton", section "The
 * Mathematical Remedy: Online Softmax Tiling") -- the same fixed merge order
 * in every workgroup of the row -- and re-reads its tile to write it
 * normalised.  Rows of more than 4096 tiles (64 MiB on the 16-byte path) get
 * the merge, in the same order, from a kernel of its own launched between
 * the two, so that it is done once per row.  This is the two-pass answer to a reduction that spans
 * workgroups ("Kernel Fusion", section "What fusion cannot fix").  Traffic is
 * two reads and one write per element; the re-read may hit L2 or the
 * Infinity Cache.  Results are those of softmax_fwd up to rounding.
 *
 * softmax_split_workspace_bytes -- device workspace bytes softmax_fwd_split
 * needs for rows x cols of `dtype` (8 bytes per tile), or -1 for bad
 * arguments.
 *
 * softmax_fwd_split -- softmax_fwd with permission to use the split path.
 *   workspace       caller-owned device memory of at least the size above,
 *                   256-byte aligned, disjoint from in and out; its contents
 *                   are scratch (overwritten, never read before written).
 *   force           0: split when rows < 1024 and a row spans two or more
 *                   tiles, otherwise run softmax_fwd's single-pass kernels
 *                   (the workspace is then unused and may be NULL); 1: always
 *                   split.  Other values: SOFTMAX_ERR_BAD_KERNEL.
 * Other arguments, layout, aliasing (in == out allowed) and errors as
 * softmax_fwd; a short or misaligned workspace is SOFTMAX_ERR_BAD_SHAPE, a
 * NULL one (when the split path runs) SOFTMAX_ERR_NULL_POINTER, one that
 * overlaps in or out SOFTMAX_ERR_OVERLAP.
 */
int64_t softmax_split_workspace_bytes(int64_t rows, int64_t cols, int dtype);
int softmax_fwd_split(const void *in, void *out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
                      void *workspace, int64_t workspace_size, int force, void *stream);

/*
 * softmax_fwd_split_noalloc -- softmax_fwd_split for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The (max, sum)
 * pairs of the split path live in a static device array of
 * SOFTMAX_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends; the call allocates nothing and calls no
 * allocating routine.  Same arguments, dispatch, kernels and results as
 * softmax_fwd_split without its workspace pair.
 *   Limit: a split call needing more than SOFTMAX_NOALLOC_SCRATCH_BYTES of
 *   workspace (softmax_split_workspace_bytes) returns
 *   SOFTMAX_ERR_SCRATCH_LIMIT before any HIP call.
 *   Sharing: every call on one GPU uses that GPU's one array.  Calls whose
 *   executions overlap on one GPU (other streams, other threads) race and
 *   may produce wrong results: serialise them.  A call reads only what its
 *   own first kernel wrote, so nothing needs clearing between calls.
 */
#define SOFTMAX_NOALLOC_SCRATCH_BYTES (1 << 20)
int softmax_fwd_split_noalloc(const void *in, void *out, int64_t rows, int64_t cols, int64_t row_stride,
                              int dtype, int force, void *stream);

/*
 * ---- Fused attention forward on the matrix cores ----
 *
 * attention_fwd -- O = softmax(scale * Q K^T) V per batch and head, with the
 * softmax fused between the two products so the nq x nk scores never reach
 * memory: the attention of "Dissecting Memory Bandwidth & SRAM Tiling in
 * Triton" (sections "Memory Hierarchy: Why Standard Attention Collapses" and
 * "Writing the Kernel in OpenAI Triton"), whose online softmax is this
 * library's merge rule applied per key block.  Both products run on
 * v_mfma_f32_32x32x16_{f16,bf16}; softmax statistics and the accumulator are
 * fp32, P is rounded to the input type before the second product.
 *   q, o        [batch][heads][nq][head_dim], dense, 16-byte aligned
 *   k, v        [batch][heads][nk][head_dim], dense, 16-byte aligned
 *   head_dim    64 or 128
 *   scale       > 0 with scale * log2(e) below 3e38 (typically 1/sqrt(head_dim));
 *               every scaled score scale * q.k * log2(e) must also be finite in
 *               fp32 (magnitude below about 3e38), or outputs may be NaN
 *   causal      0, or 1: query i keeps keys j <= i + (nk - nq) (the mask aligned
 *               to the last query); a query with no kept key gets o = 0
 *   dtype       SOFTMAX_F16 or SOFTMAX_BF16 (q, k, v and o share it)
 * o must not overlap q, k or v; k and v may be NULL when nk == 0.
 * batch * heads <= 65535, nq <= 2^30, nk * head_dim * 2 < 2^31 (K and V of
 * one head each under 2 GiB).
 * Errors: BAD_DTYPE, BAD_SHAPE (negative sizes, head_dim, misalignment, too
 * large), BAD_SCALE, NULL_POINTER, OVERLAP, HIP.  batch, heads or nq == 0
 * launches nothing.  Same asynchrony and ownership rules as softmax_fwd.
 */
int attention_fwd(const void *q, const void *k, const void *v, void *o, int64_t batch, int64_t heads,
                  int64_t nq, int64_t nk, int64_t head_dim, float scale, int causal, int dtype, void *stream);

/*
 * ---- Measurement baseline: the unfused five-operation softmax ----
 *
 * The same softmax computed as five separate kernels, each a round trip
 * through HBM: m = rowmax(x); z = x - m; num = exp(z); s = rowsum(num);
 * y = num / s -- the naive form of "GPU Kernels - Implementing and optimizing
 * Softmax" (section "Baseline & Triton Softmax kernel"), whose traffic
 * "Kernel Fusion" (section "Where the time goes in an elementwise chain")
 * counts as five reads and three writes of the tensor.  It exists so the
 * benchmark can measure what fusion saves on this machine; it is not a path
 * of softmax_fwd.  z and num are stored in the element type, m and s in fp32.
 *
 * softmax_unfused_workspace_bytes -- bytes of device workspace the baseline
 * needs for rows x cols of `dtype` (z, num, m, s), or -1 for bad arguments.
 *
 * softmax_unfused_5op -- runs the five kernels on `stream`.  Same layout and
 * aliasing rules as softmax_fwd (in == out allowed); `workspace` is caller-
 * owned device memory of at least the size above, 256-byte aligned and
 * disjoint from in and out.  Requires 16-byte-aligned in/out, and row_stride
 * and cols that are whole 16-byte accesses (else SOFTMAX_ERR_BAD_SHAPE, as for
 * a short workspace).  Rows with no finite entry give NaN, as the five
 * separate operations do.
 */
int64_t softmax_unfused_workspace_bytes(int64_t rows, int64_t cols, int dtype);
int softmax_unfused_5op(const void *in, void *out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
                        void *workspace, int64_t workspace_size, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ROW_WISE_SOFTMAX_H */
