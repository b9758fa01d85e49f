/*
 * tb.h -- C ABI of libtb.so, the ternary-weight int8 FFN decode path for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation, after "perf(bonsai): decode and small packed batches read
 * the FFN from a ternary copy through a dp4a GEMV" (sparkinfer PR #1154),
 * Summary and commit message:
 *   - decode reads each FFN's stored ternary weight blocks;
 *   - the activation is rotated by a Hadamard transform and quantised to
 *     int8 once; the gate and up matrices both read that one int8 vector;
 *   - an integer dot-product GEMV folds the per-block scales into each
 *     block's integer sum;
 *   - a packed step of up to 8 rows gives every row exactly the bytes it gets
 *     alone.
 * Formats: the bonsai-edge-serve README (model list, "kernels/") names
 * ternary weights in groups of 128, and a 1-bit variant.
 *
 * Conventions for every entry point
 *   Memory   All array pointers are DEVICE pointers, owned by the caller,
 *            16-byte aligned, row-major and contiguous. tb_matrix structs and
 *            the tb_matrix pointers are HOST memory; they are read during the
 *            call only. The library allocates no device memory and keeps no
 *            pointer after it returns.
 *   State    The only state is a process-wide table, filled on a device's
 *            first call and guarded by a mutex, of that device's LDS limit and
 *            compute-unit count, and the kernels whose LDS limit has been
 *            raised. It never changes a result. Calls from several host
 *            threads are safe.
 *   Rows     m is the number of activation rows, 1 <= m <= 8. Rows are
 *            independent. Row r's outputs are bit-identical for every m and
 *            for every position r in the batch.
 *   Shapes   k is a multiple of 128 (k >= 128); n >= 1. nb = k / 128.
 *   Stream   stream is a hipStream_t passed as void*; 0 is the null stream.
 *            Work is enqueued on it asynchronously. Inputs must stay valid,
 *            and outputs unread, until the stream has run it.
 *   Errors   Arguments are checked before anything is launched. A bad value
 *            returns TB_EINVAL, a misaligned pointer TB_EALIGN, an input that
 *            overlaps an output TB_EINVAL, and a shape the library cannot run
 *            TB_EUNSUPPORTED. In all of these cases nothing is enqueued. A HIP
 *            error at launch returns TB_EHIP. A fault while the kernel runs
 *            surfaces at the caller's next synchronisation. Nothing is
 *            printed, nothing aborts, and no C++ exception crosses the ABI.
 *   Numbers  Inputs must be finite. Results are deterministic: the same
 *            inputs give the same bytes on every run.
 */
#ifndef TB_H
#define TB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TB_ABI_VERSION 6
#define TB_BLOCK 128
#define TB_MAX_ROWS 8
#define TB_MAX_BATCH_ROWS 32

enum tb_status {
    TB_OK = 0,
    TB_EINVAL = -1,       /* bad shape, null pointer, unknown format, aliasing */
    TB_EALIGN = -2,       /* a pointer is not 16-byte aligned */
    TB_EUNSUPPORTED = -3, /* valid arguments the library cannot run (e.g. LDS too small) */
    TB_EHIP = -4,         /* the HIP runtime reported an error */
    TB_ESCRATCH = -5      /* input larger than the library's static scratch (tb_ffn_down_noalloc) */
};

enum tb_format {
    /* 2-bit ternary codes. Weight i of a row is the 2-bit field at byte i>>2,
     * bits 2*(i&3) and 2*(i&3)+1, least significant first. Code 0 -> 0,
     * 1 -> +1, 2 -> -1, 3 -> 0. codes: uint8[n][nb][32]. */
    TB_FMT_TERNARY2 = 0,
    /* 1-bit signs. Weight i is bit i&7 of byte i>>3; 1 -> +1, 0 -> -1.
     * codes: uint8[n][nb][16]. */
    TB_FMT_SIGN1 = 1,
    /* The same signs, rows interleaved by four for the lookup-table GEMV
     * (bonsai-edge-serve README, kernels/ section: a 1-bit lookup-table kernel
     * needs a row-interleaved layout). n % 4 == 0. codes: uint32[n/4][nb][16],
     * byte r of word j = byte j of row 4*(quad)+r's block; scales:
     * uint16[n/4][nb][4]. Made by tb_sign_interleave; taken by tb_gemv_ternary
     * and tb_gemv_block_sums (and their _batch forms) for m <= 2 only. */
    TB_FMT_SIGN1_RI4 = 2
};

/* One weight matrix with n output rows and k inputs.
 * scales: uint16[n][nb], IEEE binary16 bit patterns, one per 128-weight
 * block. The dequantised weight is W[j][i] = scale[j][i/128] * t(j, i).
 * The kernels read scales as aligned 4-byte words; when n * nb is odd the
 * 2 bytes after the array (in the same aligned word) are read and ignored.
 * Each of codes and scales must be smaller than 2 GiB (else TB_EUNSUPPORTED). */
typedef struct tb_matrix {
    const void *codes;
    const uint16_t *scales;
    int32_t n;
    int32_t k;
    int32_t fmt; /* enum tb_format */
} tb_matrix;

/* Rotate and quantise activation rows: the step that turns the activation into
 * its rotated int8 copy (PR #1154, commit message).
 * For every row r and 128-block b, with v = x[r][128b .. 128b+127]:
 *   u = H v       unnormalised Walsh-Hadamard transform, H[i][j] =
 *                 (-1)^popcount(i&j). Butterfly stages of span 1, 2, ..., 64
 *                 in that order, each (a, b) -> (a+b, a-b) in fp32.
 *   amax = max |u_i|. If amax == 0, q = 0 and dq = 0.
 *   Otherwise q_i = rint(u_i * (127/amax)) (fp32, ties to even) and
 *   dq = amax * fp32(1/(127*sqrt(128))).
 * So q*dq approximates (H/sqrt(128)) v, an orthonormal rotation of v.
 *   x  float [m][k]     input
 *   q  int8  [m][k]     output
 *   dq float [m][k/128] output */
int tb_rotate_quant_i8(const float *x, int m, int k, int8_t *q, float *dq, void *stream);

/* Ternary (or sign) GEMV: integer dot products per 128-weight block, each
 * block's scales folded into its integer sum, and a fixed lane tree per row
 * (PR #1154, commit message).
 *   isum[r][j][b] = sum_i t(j, 128b+i) * q[r][128b+i]          (int32, exact)
 *   y[r][j]       = sum_b scale[j][b] * dq[r][b] * isum[r][j][b]  (fp32 fold)
 *   w  matrix with w->k inputs, w->n outputs, fmt TERNARY2 or SIGN1
 *   q  int8 [m][w->k], dq float [m][w->k/128]   (from tb_rotate_quant_i8)
 *   y  float [m][w->n] output
 * The fp32 fold is within 1e-4 * sum_b |term_b| of the exact value. */
int tb_gemv_ternary(const tb_matrix *w, const int8_t *q, const float *dq, int m, float *y,
                    void *stream);

/* Gate and up GEMVs from one shared int8 copy, then the SiLU gate. The two
 * projections read the same rotated int8 activation, made once per step
 * (PR #1154, commit message):
 *   g = gemv(wg, q, dq), u = gemv(wu, q, dq), h[r][j] = silu(g) * u with
 *   silu(z) = z / (1 + exp(-z)).
 *   wg, wu  same n, k and fmt
 *   h       float [m][wg->n] output */
int tb_ffn_gateup_silu(const tb_matrix *wg, const tb_matrix *wu, const int8_t *q,
                       const float *dq, int m, float *h, void *stream);

/* Gate/up from the fp32 activation: tb_rotate_quant_i8(x) into qx, dqx, then
 * tb_ffn_gateup_silu on them, as one call. The rotated int8 copy is made once
 * per step and shared by the two projections (PR #1154, commit message). For
 * up to 4 rows on the dot-product kernel with m * k/128 <= 128 (two blocks per
 * 16-lane group of a workgroup; at k = 5120, m <= 3) every workgroup makes its
 * own copy in LDS while its first weight loads are in flight, which saves the
 * separate launch, and workgroup 0 writes the copy to qx, dqx; otherwise the
 * call runs the two launches. Results are bit-identical to the two calls
 * (same rotation arithmetic, same fold).
 *   x    float [m][wg->k]     input, 16-byte aligned
 *   qx   int8  [m][wg->k]     output: rotquant(x) codes
 *   dqx  float [m][wg->k/128] output: their block scales
 *   h    float [m][wg->n]     output
 * 1 <= m <= 8; the outputs may not overlap one another or the inputs. */
int tb_ffn_gateup_silu_x(const tb_matrix *wg, const tb_matrix *wu, const float *x, int m,
                         int8_t *qx, float *dqx, float *h, void *stream);

/* Down projection of the FFN: rotate and quantise h exactly like
 * tb_rotate_quant_i8, into caller-owned workspace, then the GEMV. The pages'
 * int8 scratch is allocated with the weight copy, never as hidden static
 * memory (PR #1154, Summary), so here the caller passes it in.
 * Where tb_ffn_gateup_silu_x would rotate inside its launch (up to 4 rows on
 * the dot-product kernel, m * k/128 <= 128; not at k = 17408) the rotation of
 * h runs inside the GEMV's launch; otherwise, and always in the batch
 * variant, the two steps are separate launches. Either way the results are
 * the same bits.
 *   h       float [m][wd->k]    input (the output of tb_ffn_gateup_silu)
 *   qh_ws   int8  [m][wd->k]    workspace; holds rotquant(h) on return
 *   dqh_ws  float [m][wd->k/128] workspace; holds its scales on return
 *   y       float [m][wd->n]    output */
int tb_ffn_down(const tb_matrix *wd, const float *h, int m, int8_t *qh_ws, float *dqh_ws,
                float *y, void *stream);

/* GEMV of fp32 rows: tb_rotate_quant_i8(x) into qx, dqx, then tb_gemv_ternary
 * on them, as one call; the same operation and code as tb_ffn_down, for any
 * projection whose input arrives in fp32 (the attention projections of the
 * same model). Where the rows allow it (as for tb_ffn_gateup_silu_x) x is
 * rotated inside the GEMV's launch; results are bit-identical to the two
 * calls.
 *   x    float [m][w->k]     input, 16-byte aligned
 *   qx   int8  [m][w->k]     output: rotquant(x) codes
 *   dqx  float [m][w->k/128] output: their block scales
 *   y    float [m][w->n]     output
 * 1 <= m <= 8; the outputs may not overlap one another or the inputs. */
int tb_gemv_ternary_x(const tb_matrix *w, const float *x, int m, int8_t *qx, float *dqx, float *y,
                      void *stream);

/* Test export: the per-block integer sums, before the scale fold, computed by
 * the integer core that production runs:
 *   m <= 4, or k/128 not a multiple of 2 (ternary) or 4 (sign): the dot-product
 *     core (v_dot4), which tb_gemv_ternary and tb_ffn_gateup_silu run for those m;
 *   m >= 5 otherwise: the matrix-core core (v_mfma_i32_16x16x64_i8), which
 *     tb_ffn_gateup_silu runs from m = 5 on and tb_gemv_ternary (so tb_ffn_down)
 *     from m = 6 (ternary) or m = 7 (sign) on.
 * For a single GEMV at m = 5 (ternary) or m = 5, 6 (sign) production runs the
 * dot-product core, which this export runs at m <= 4: the same code, templated
 * on m.
 *   isum int32 [m][w->n][w->k/128] output; m * n * (k/128) * 4 must be below
 *   2 GiB (else TB_EUNSUPPORTED). */
int tb_gemv_block_sums(const tb_matrix *w, const int8_t *q, int m, int32_t *isum, void *stream);

/* Row-interleave a TB_FMT_SIGN1 matrix (n % 4 == 0) into TB_FMT_SIGN1_RI4:
 * codes_ri receives n*k/8 bytes, scales_ri n*(k/128) fp16 values, both
 * caller-owned device buffers, 16-byte aligned, overlapping nothing. The
 * interleaved matrix is {codes_ri, scales_ri, n, k, TB_FMT_SIGN1_RI4}. With
 * it tb_gemv_ternary runs a lookup-table kernel (v_perm_b32 looks up the
 * sums of a pair of activations for four rows at once) whose y is
 * bit-identical to the bit-mask kernel on the original matrix; m > 2 returns
 * TB_EUNSUPPORTED (the tables of one row take 32 registers per lane), and
 * the gate/up, down and fused calls return TB_EUNSUPPORTED for this layout. */
int tb_sign_interleave(const tb_matrix *w, void *codes_ri, uint16_t *scales_ri, void *stream);

/* ---- Batches above 8 rows ------------------------------------------------
 * The same five operations for 1 <= m <= TB_MAX_BATCH_ROWS (32) rows: for
 * concurrent decodes beyond the packed steps of 8 that the calls above take
 * (PR #1154, Proof of speedup, where the ternary copy left 16 and 32
 * concurrent requests unchanged; bonsai-edge-serve README, speculative-decoding
 * section, on an integer-dot batch kernel for these formats). Arguments,
 * layouts, outputs and errors are those of the call without the suffix, with
 * m up to 32; each row's outputs are bit-identical to the same row run alone
 * through either family.
 * The rows run as balanced chunks: chunks of up to 16 rows on the matrix-core
 * kernel with all 16 B columns live (one read of the weights per chunk) where
 * the shape's activation and step partials fit the device's LDS and k/128 is a
 * multiple of 2 (ternary) or 4 (sign); otherwise chunks of up to 8 rows on the
 * kernels of the calls above. Ternary gate/up of 17 to 32 rows runs in one
 * launch (two 16-column groups, k staged in two phases) where its LDS plan
 * fits. At hidden 5120, intermediate 17408: gate/up takes the whole batch
 * (ternary) or 16 rows per chunk (sign), the down GEMV 8 (see
 * tb_ffn_down_split_batch for a down stage that reads its weights once).
 * tb_gemv_block_sums_batch: (chunk rows) * n * (k/128) * 4 must be below
 * 2 GiB. */
int tb_rotate_quant_i8_batch(const float *x, int m, int k, int8_t *q, float *dq, void *stream);
int tb_gemv_ternary_batch(const tb_matrix *w, const int8_t *q, const float *dq, int m, float *y,
                          void *stream);
int tb_ffn_gateup_silu_batch(const tb_matrix *wg, const tb_matrix *wu, const int8_t *q,
                             const float *dq, int m, float *h, void *stream);
int tb_ffn_down_batch(const tb_matrix *wd, const float *h, int m, int8_t *qh_ws, float *dqh_ws,
                      float *y, void *stream);
int tb_gemv_block_sums_batch(const tb_matrix *w, const int8_t *q, int m, int32_t *isum,
                             void *stream);

/* ---- Down stage split over k -------------------------------------------
 * tb_ffn_down with a caller workspace that lets the down stage run split over k
 * as well as over rows (PR #1154, Summary and commit message: h is rotated and
 * quantised to int8, then the down matrix's blocks are multiplied against that
 * copy). From 4 rows on, on the matrix cores: each workgroup of the first
 * launch takes one step (8 ternary or 16 sign blocks) of one row group. It
 * rotates and quantises those blocks of h itself (the rotate-quantise
 * arithmetic, bit for bit) and streams the group's weights at that step, and
 * each row's step partial goes to ws. A second, small launch adds every row's
 * partials in step order. That is the fold of tb_ffn_down, so y, qh and dqh are
 * bit-identical to tb_ffn_down on the same inputs. What it saves is the
 * separate rotation launch and the staging of all of rotquant(h) in every CU.
 * It takes the split from 4 rows while tb_ffn_down's GEMV would run on the
 * dot-product kernel (ternary up to 5 rows, sign up to 6), and for more rows only
 * when k >= 8192, where the unsplit kernel stages m * k codes in every CU (the
 * down stage of the FFN). Otherwise (where the split measured slower), or where
 * its plan does not apply (k/128 not a multiple of 2 (ternary) or 4 (sign)), the
 * call runs tb_ffn_down and leaves ws untouched.
 *   h    float [m][wd->k]     input
 *   qh   int8  [m][wd->k]     output: rotquant(h) codes
 *   dqh  float [m][wd->k/128] output: their block scales
 *   y    float [m][wd->n]     output
 *   ws   device workspace of at least tb_ffn_down_split_workspace_bytes(wd, m)
 *        bytes, 16-byte aligned: the step partials, float [steps][m][wd->n],
 *        steps = ceil(k / 1024) for ternary and ceil(k / 2048) for sign. It needs
 *        no initialisation; calls that share one must not overlap in time.
 * 1 <= m <= 8; the format must not be TB_FMT_SIGN1_RI4. Outputs and workspace
 * may not overlap one another or the inputs. Returns TB_EINVAL for a
 * workspace that is too small. */
int tb_ffn_down_split(const tb_matrix *wd, const float *h, int m, int8_t *qh, float *dqh,
                      float *y, void *ws, size_t ws_bytes, void *stream);
/* Workspace bytes of tb_ffn_down_split for m rows; 0 for invalid arguments. */
size_t tb_ffn_down_split_workspace_bytes(const tb_matrix *wd, int m);

/* tb_ffn_down_split for 1 <= m <= TB_MAX_BATCH_ROWS (32) rows, the down stage
 * of the batches above 8 rows (see tb_ffn_down_batch for the pages' passages).
 * Up to 8 rows it is tb_ffn_down_split. From 9 rows, when k >= 8192, it runs on
 * the matrix-core kernel with all 16 B columns live, split over k as above (one
 * step of one row group per workgroup, h rotated and quantised inside), then one
 * fold launch for the batch. Ternary: one launch for the whole batch, whose B
 * operands hold 16 rows, or 32 in two column groups sharing each decoded weight
 * operand, so the down weights are read once. Sign: balanced chunks of up to 16
 * rows, one launch each. tb_ffn_down_batch, whose 16-row kernel cannot stage
 * k = 17408 codes per row in a CU, reads them once per 8 rows. Otherwise (k < 8192,
 * or the plan does not fit the device) the call runs tb_ffn_down_batch and leaves
 * ws untouched. Arguments, layouts, outputs, workspace and errors are those of
 * tb_ffn_down_split with m up to 32; each row's y, qh and dqh are bit-identical
 * to tb_ffn_down on that row alone. */
int tb_ffn_down_split_batch(const tb_matrix *wd, const float *h, int m, int8_t *qh, float *dqh,
                            float *y, void *ws, size_t ws_bytes, void *stream);
/* Workspace bytes of tb_ffn_down_split_batch for m rows (1 ... 32); 0 for
 * invalid arguments. */
size_t tb_ffn_down_split_batch_workspace_bytes(const tb_matrix *wd, int m);

/* ---- No allocation -------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation):
 * tb_ffn_down without the workspace arguments. rotquant(h) and its scales go
 * to a device array inside the library (TB_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the first call on that GPU until the process ends), so the call
 * allocates nothing. Same arguments, kernels and outputs as tb_ffn_down; y is
 * bit-identical to it.
 *   Limit    round_up(m * k, 256) + m * (k/128) * 4 <= TB_NOALLOC_SCRATCH_BYTES
 *            (for m = 8: k up to 126,976); larger inputs return TB_ESCRATCH and
 *            enqueue nothing.
 *   Sharing  Every call on one GPU uses that GPU's one array, which keeps the
 *            last call's contents. Calls that overlap in time on one GPU (on
 *            different streams, or from several host threads) race on it and
 *            must be serialised by the caller. Nothing in it needs clearing:
 *            each call overwrites what it reads.
 *   First call on a GPU looks up the array's device address (no allocation). */
#define TB_NOALLOC_SCRATCH_BYTES (1u << 20)
int tb_ffn_down_noalloc(const tb_matrix *wd, const float *h, int m, float *y, void *stream);

/* ---- Fused FFN layers ----------------------------------------------------
 * One launch runs num_layers whole FFN layers of the same shape: for each
 * layer, exactly tb_rotate_quant_i8(x) -> tb_ffn_gateup_silu ->
 * tb_ffn_down (the stages of PR #1154's decode step, Summary and commit
 * message). Outputs are bit-identical to those three calls. One workgroup per
 * compute unit stays resident for all layers and streams the weights without
 * pausing at kernel boundaries; layers run strictly one after another (layer
 * l+1 starts after every output of layer l is written).
 *   layers   host array of num_layers weight sets: gate, up [inter x hidden],
 *            down [hidden x inter], one fmt; inter a multiple of 128.
 *   x        float [num_layers][m][hidden] (one input per layer), or with
 *            TB_FFN_CHAIN float [m][hidden]: layer l+1 then takes layer l's y.
 *   y        float [num_layers][m][hidden] outputs.
 *   ws       device workspace of at least tb_ffn_workspace_bytes(m, hidden,
 *            inter) bytes, 16-byte aligned, initialised with
 *            tb_ffn_workspace_init before its first use and again whenever m,
 *            hidden or inter change. It holds the data exchanged between
 *            workgroups (h, rotquant(h) and y, each value stored with a tag
 *            naming its launch and layer) and the synchronisation words; every
 *            call leaves it ready for the next. Calls that share a workspace
 *            must not overlap in time.
 * Synchronisation between workgroups waits a bounded time (the spin limit of
 * tb_ffn_workspace_init; 0 selects 100 ms). If a wait runs out, for instance
 * because other work occupies compute units so that not all workgroups can
 * be resident, the call abandons its work (outputs undefined) and sets a
 * sticky error in the workspace, read with tb_ffn_workspace_error; later
 * calls on that workspace do nothing until it is initialised again. */
typedef struct tb_ffn_weights {
    tb_matrix gate, up, down;
} tb_ffn_weights;

#define TB_FFN_CHAIN 1u

size_t tb_ffn_workspace_bytes(int m, int hidden, int inter);  /* 0 for bad arguments */
int tb_ffn_workspace_init(void *ws, size_t ws_bytes, uint32_t spin_ticks, void *stream);
int tb_ffn_layers(const tb_ffn_weights *layers, int num_layers, const float *x, int m,
                  unsigned flags, void *ws, size_t ws_bytes, float *y, void *stream);
/* Blocking: synchronises with the device and returns the sticky error word
 * (0 = none) in *error. */
int tb_ffn_workspace_error(const void *ws, int *error);

/* Static description of a status code; never NULL. */
const char *tb_status_str(int status);

/* TB_ABI_VERSION of the built library. */
int tb_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TB_H */
