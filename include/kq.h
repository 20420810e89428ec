/*
 * kq.h -- C ABI of the K-quant decode GEMV library for AMD MI355X (gfx950).
 *
 * The operation is the decode-step matrix-vector product over GGUF K-quant
 * weights,
 *
 *     y[b, r] = sum_k dequant(W)[r, k] * x[b, k]        for b < batch <= 16,
 *
 * where every generated token streams the whole quantised decoder through it
 * once.  Sources for what is computed:
 *   - Q4_K / Q5_K / Q6_K super-blocks executed natively on the GPU, with a
 *     backend-specific repack: daily.dev summary of the ExecuTorch announcement,
 *     Q&A "How does ExecuTorch export Muse Glimmer GGUF checkpoints for CUDA and
 *     Apple Silicon?".
 *   - decode priced as weight bytes streamed per token: "Muse-Glimmer-30B (text
 *     decoder) - Apple Core AI", decode table and the paragraph after it.
 *   - batch 1 per exported method: "Muse Glimmer 30B - ExecuTorch PTE" card,
 *     section "Runtime limitations"; batch 1 through 8: SGLang Day-0 post,
 *     paragraph on the seven-platform sweep.
 *   - projections that read the same hidden state folded into one product:
 *     Core AI card, section "The architecture, and what the port had to do
 *     about it" (qkvg_proj, 4 GEMMs -> 1).
 *
 * Dequantisation (one rounding to fp32 of an exact value):
 *   Q4_K, Q5_K: w = d * sc_g * q - dmin * m_g    (sub-blocks g of 32 weights)
 *   Q6_K      : w = d * sc_g * (q - 32)          (sub-blocks g of 16 weights)
 *
 * Rounding of y: the quants enter the dot products as exact bf16 operands
 * (q, or 4(q - 32) for Q6_K, with no offset), so each sub-block's sum is
 * rounded relative to its own terms and y is within 1e-4 * sum_k |w x| of the
 * exact product, also on rows whose sum comes from a single weight.  The one
 * precondition: Q4_K/Q5_K add the two exact terms d*sc*sum(q x) and
 * dmin*m*sum(x) per sub-block in fp32, so where they cancel for EVERY element
 * of a sub-block (w = 0 with q and m nonzero, a legal but degenerate encoding)
 * the error is bounded by 2^-19 * sum (|d sc q| + |dmin m|) |x| over that
 * sub-block instead.
 *
 * Conventions for every entry point:
 *   - Pointers named w, gguf, out, x, y are DEVICE pointers owned by the caller;
 *     array-of-pointer and array-of-size arguments of kq_gemv_multi are HOST
 *     arrays read during the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued asynchronously; the call returns once it is enqueued.
 *   - Arguments are validated on the host first; on any error the call returns
 *     a non-zero KQ_ERR_* code and enqueues nothing.  A failed launch returns
 *     KQ_ERR_HIP.  No C++ exception crosses the boundary.
 *   - `cols` (K) must be a positive multiple of 256; `rows` (M) >= 1.
 *   - The library allocates no memory on any GEMV call path and keeps no
 *     mutable global state.  GEMV calls whose outputs are split across
 *     workgroups need device scratch (partial sums of K-split row tiles,
 *     arrival counters, the heads' sums of squares of a head-norm epilogue):
 *     the CALLER passes it as a workspace, `ws` (device, 16-byte aligned) of
 *     `ws_bytes` bytes.  KQ_WORKSPACE_BYTES is enough for any call;
 *     kq_gemv_workspace_bytes gives the exact need of one call.  Its first
 *     64 KiB are counters that must be zero before the first use
 *     (kq_workspace_init) and that every call leaves zero again.  One
 *     workspace serves any number of calls ordered on one stream; calls that
 *     may overlap in time (unordered streams, threads) need distinct
 *     workspaces, exactly as they need distinct outputs.  A NULL, misaligned
 *     or too small workspace returns KQ_ERR_WORKSPACE and enqueues nothing.
 *     Every call is then thread-safe and may be captured in a HIP graph.
 */
#ifndef KQ_H
#define KQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KQ_ABI_VERSION 2

/* weight formats */
#define KQ_Q4_K 1
#define KQ_Q5_K 2
#define KQ_Q6_K 3

/* activation formats: fp32, or bf16 (bit patterns, 2 bytes per element).
 * fp32 activations are carried as two bf16 terms, hi = bf16(x) and
 * lo = bf16(x - hi), which give x to within 2^-18 |x|; the products of both run
 * as a bf16 batch of twice the size.  The GEMV bound (1e-4 * sum |w x|) holds for
 * rows whose largest |x| is at least 2^-100 (below, lo falls among bf16's
 * subnormals and loses bits) and at most 2^100. */
#define KQ_X_F32 0
#define KQ_X_BF16 1

/* batch rows per call: up to 16 with bf16 activations (one speculative-verify
 * block: the drafter proposes blocks of 16 tokens and the runner accepts block
 * lengths 2..16, "Muse Glimmer 30B - ExecuTorch PTE" card, paragraph "Faster
 * Generation Through Speculative Decoding" and "Adjustments per variant"), up
 * to 8 with fp32 */
#define KQ_MAX_BATCH 16
#define KQ_MAX_BATCH_F32 8
#define KQ_MAX_PROJ 8

/* epilogues (what a launch does with a finished output before storing it) */
#define KQ_EPI_NONE 0
#define KQ_EPI_SWIGLU 1    /* silu(gate) * up, see kq_gemv_swiglu */
#define KQ_EPI_SIGMOID 2   /* y = 1 / (1 + exp(-(W x))): the attention output gate */
#define KQ_EPI_RESIDUAL 3  /* y = y + W x: y holds the residual stream on entry */
#define KQ_EPI_HEADNORM 4  /* weight-less RMSNorm of each KQ_HEAD_ROWS outputs (the Q and K heads) */
#define KQ_HEAD_ROWS 128   /* outputs per head of a KQ_EPI_HEADNORM segment (head_dim) */

/* status codes */
#define KQ_OK 0
#define KQ_ERR_NULL 1   /* a required pointer is NULL */
#define KQ_ERR_SHAPE 2  /* rows < 1, cols not a positive multiple of 256, ldx < cols, ldy < rows, ... */
#define KQ_ERR_ALIGN 3  /* w / x not 16-byte aligned, y not 4-byte aligned, or row stride of x not 16 B */
#define KQ_ERR_BATCH 4  /* batch outside 1..KQ_MAX_BATCH (KQ_MAX_BATCH_F32 for fp32 x), or n outside 1..KQ_MAX_PROJ */
#define KQ_ERR_TYPE 5   /* unknown weight or activation format */
#define KQ_ERR_HIP 6    /* a HIP runtime call or kernel launch failed */
#define KQ_ERR_NOMEM 7  /* scratch allocation failed */
#define KQ_ERR_RANGE 8  /* problem too large for 32-bit tile indexing */
#define KQ_ERR_TIMEOUT 9 /* a chain step's wait for the previous step gave up (kq_chain_status) */
#define KQ_ERR_DEVICE 10 /* a chain was run with another device current than the one it was made on */
#define KQ_ERR_WORKSPACE 11 /* workspace NULL, not 16-byte aligned, or smaller than the call needs */

/* Workspace bytes that suffice for any GEMV call (69 MiB; most calls need far
 * less, see kq_gemv_workspace_bytes). */
#define KQ_WORKSPACE_BYTES 72417280u

/* Version of this ABI (KQ_ABI_VERSION). */
int kq_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char *kq_status_str(int status);

/*
 * Check that `device` (the HIP ordinal) exists and can be queried, and look up
 * the device address of its kq_gemv_fused_noalloc scratch (otherwise done at
 * that entry point's first call on the device).  Allocates nothing.  Returns
 * KQ_OK, else KQ_ERR_DEVICE / KQ_ERR_HIP.
 */
int kq_init(int device);

/*
 * Exact workspace bytes of one GEMV call with these shapes and options on the
 * current device (the launch geometry depends on its CU count), as
 * kq_gemv_fused takes them: epi may be NULL, rms_eps as there.  0 if the
 * arguments are invalid.  Host-only query; allocates nothing.
 */
size_t kq_gemv_workspace_bytes(int type, int n, const int64_t *rows, int64_t cols, int xtype, int batch,
                               const int32_t *epi, float rms_eps);

/*
 * Prepare a workspace for its first use: zero its counter block (the first
 * 64 KiB) with a kernel on `stream` (no memset node, so it may be captured).
 * bytes >= 64 KiB and ws 16-byte aligned, else KQ_ERR_WORKSPACE.
 */
int kq_workspace_init(void *ws, size_t bytes, void *stream);

/*
 * Size in bytes of the repacked form of a rows x cols matrix of `type`, or 0 if
 * the arguments are invalid.  Host-only; makes no HIP call.
 *
 * Layout (all offsets in bytes): rows are grouped in tiles of 64 (the last tile
 * zero-padded).  Tile t, super-block column c starts at ((t * cols/256) + c) *
 * 64 * S, S = 144 / 176 / 210.  Inside it, 16-byte chunk k of the super-block
 * of row 64*t + r is at k*1024 + 16*r, so one 64-lane wavefront reads each
 * chunk as one contiguous 1 KiB; Q6_K's fp16 d of row r follows all chunks at
 * 13*1024 + 2*r.  The chunk contents re-order each super-block's bits (scale
 * and min bytes beside their quants) without changing the byte count.
 */
size_t kq_repacked_bytes(int type, int64_t rows, int64_t cols);

/*
 * Repack GGUF super-blocks into the layout above.
 *   gguf : device, rows * cols/256 super-blocks in GGUF row-major order
 *          (144 / 176 / 210 bytes each); any alignment.
 *   out  : device, kq_repacked_bytes(type, rows, cols) bytes, 16-byte aligned.
 * One-time, off the per-token path (the "repacked ... kernels" of the daily.dev
 * summary's GGUF Q&A).
 */
int kq_repack(int type, int64_t rows, int64_t cols, const void *gguf, void *out, void *stream);

/*
 * y[b*ldy + r] = sum_k dequant(W)[r, k] * x[b*ldx + k], r < rows, b < batch.
 *   w    : repacked Q4_K (resp. Q5_K, Q6_K) weights from kq_repack with the same
 *          rows and cols (not checked: it would need a device read).
 *   x    : fp32 or bf16 activations, batch rows of stride ldx elements; 16-byte
 *          aligned and ldx * element size a multiple of 16.
 *   y    : fp32 output, batch rows of stride ldy >= rows; 4-byte aligned.
 *   ws, ws_bytes : the caller's workspace (see the conventions above).
 * Deterministic: the same inputs give bitwise the same y on every run.
 */
int kq_gemv_q4k(const void *w, int64_t rows, int64_t cols, const void *x, int xtype, int64_t ldx, int batch,
                float *y, int64_t ldy, void *ws, size_t ws_bytes, void *stream);
int kq_gemv_q5k(const void *w, int64_t rows, int64_t cols, const void *x, int xtype, int64_t ldx, int batch,
                float *y, int64_t ldy, void *ws, size_t ws_bytes, void *stream);
int kq_gemv_q6k(const void *w, int64_t rows, int64_t cols, const void *x, int xtype, int64_t ldx, int batch,
                float *y, int64_t ldy, void *ws, size_t ws_bytes, void *stream);

/*
 * n projections of one type that read the same x (QKV, gate+up), in ONE launch:
 * y[i][b*ldy[i] + r] = sum_k dequant(W_i)[r, k] * x[b*ldx + k], r < rows[i].
 *   w, rows, y, ldy : host arrays of n entries (device pointers in w and y).
 * Same per-matrix rules as kq_gemv_q4k.  1 <= n <= KQ_MAX_PROJ.
 */
int kq_gemv_multi(int type, int n, const void *const *w, const int64_t *rows, int64_t cols, const void *x, int xtype,
                  int64_t ldx, int batch, float *const *y, const int64_t *ldy, void *ws, size_t ws_bytes,
                  void *stream);

/*
 * out[r*ldo + k] = dequant(W)[r, k] as fp32 (the single correctly rounded value
 * of the exact dequantised weight), from the repacked layout.  ldo >= cols,
 * out 4-byte aligned.  Used to check the repack and unpack bit-exactly.
 */
int kq_dequant(int type, const void *w, int64_t rows, int64_t cols, float *out, int64_t ldo, void *stream);

/*
 * Measurement: read `bytes` (a multiple of 16) of device memory at p
 * (16-byte aligned) once, with the GEMV's own loads (128-bit nontemporal
 * buffer loads, many in flight) and no arithmetic.  Its rate is the
 * achievable HBM read rate that the weight streaming is held against (a
 * decode step costs its weight bytes: "Muse-Glimmer-30B (text decoder) -
 * Apple Core AI", decode table and the paragraph after it).  `sink`: one
 * device word, written only if the xor of all data equals a fixed value, so
 * that the loads cannot be dropped.  bytes == 0 enqueues nothing.
 */
int kq_stream_read(const void *p, size_t bytes, uint32_t *sink, void *stream);

/*
 * kq_gemv_multi with the work either side of the projections folded into the
 * launch ("Muse-Glimmer-30B (text decoder) - Apple Core AI", section "The
 * architecture, and what the port had to do about it"):
 *
 * Before: rms_eps > 0 normalises every activation row first with a weight-less
 * RMSNorm (the card puts one on the embedding output and on Q/K),
 *     y[i][b*ldy + r] = sum_k dequant(W_i)[r, k] * x[b, k] / sqrt(mean_k x[b, k]^2 + rms_eps).
 * The launch computes sum_k x[b, k]^2 alongside the staging of x and scales the
 * finished dot products, which is the same quantity.  rms_eps == 0: no
 * normalisation; negative, infinite or NaN: KQ_ERR_SHAPE.
 *
 * After: epi (host array of n codes, or NULL for all KQ_EPI_NONE) gives each
 * segment's epilogue:
 *   KQ_EPI_SIGMOID  y = 1 / (1 + exp(-y)): the sigmoid output gate read from the
 *                   same hidden state as Q/K/V, the fourth segment of the fused
 *                   qkvg launch;
 *   KQ_EPI_RESIDUAL y = r + y, r read from y[i][b*ldy + r] before it is written:
 *                   the residual add that closes the attention and feed-forward
 *                   blocks around the O and down projections (a segment's y must
 *                   not overlap another segment's);
 *   KQ_EPI_HEADNORM the card's weight-less RMSNorm on Q/K: every KQ_HEAD_ROWS
 *                   consecutive outputs of the segment form a head, and
 *                   y = v / sqrt(mean over the head of v^2 + head_eps) per batch
 *                   row.  rows[i] must be a multiple of KQ_HEAD_ROWS and
 *                   head_eps finite and > 0 (else KQ_ERR_SHAPE); a launch with
 *                   such a segment has at most 8192 tiles of 64 rows in total
 *                   (else KQ_ERR_RANGE).  head_eps is ignored without one;
 *   KQ_EPI_SWIGLU   n = 1 only, w from kq_repack_swiglu and rows[0] = inter:
 *                   as kq_gemv_swiglu.
 *
 * bf16 copies: y16 (host array of n device pointers, or NULL) names for each
 * segment an optional second output, y16[i][b*ldy16[i] + r] = the bf16 nearest
 * (round to nearest even) to the fp32 value written to y[i], so that a product
 * that reads this output can take bf16 activations (ldy16[i] >= rows[i], 2-byte
 * aligned; a NULL entry: none).
 * Otherwise as kq_gemv_multi; KQ_ERR_TYPE for an unknown code.
 */
int kq_gemv_fused(int type, int n, const void *const *w, const int64_t *rows, int64_t cols, const void *x, int xtype,
                  int64_t ldx, int batch, float *const *y, const int64_t *ldy, void *const *y16, const int64_t *ldy16,
                  const int32_t *epi, float rms_eps, float head_eps, void *ws, size_t ws_bytes, void *stream);

/*
 * kq_gemv_fused for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments without (ws, ws_bytes) and the same results bitwise.  Its
 * workspace is a static array of KQ_NOALLOC_SCRATCH_BYTES (8 MiB) in the
 * library's device code, one copy per GPU, which each GPU holds until the
 * process ends; the entry point calls no hipMalloc, hipFree or allocating
 * routine.  A call whose workspace need (kq_gemv_workspace_bytes) exceeds it
 * is refused with KQ_ERR_WORKSPACE, enqueueing nothing.  Each call first
 * clears the array's counter block with a kernel on `stream`.  Every call on
 * one GPU shares that GPU's array: calls that may overlap in time on one GPU
 * (unordered streams, threads) race and give wrong results; order them.
 */
#define KQ_NOALLOC_SCRATCH_BYTES 8388608u
int kq_gemv_fused_noalloc(int type, int n, const void *const *w, const int64_t *rows, int64_t cols, const void *x,
                          int xtype, int64_t ldx, int batch, float *const *y, const int64_t *ldy,
                          void *const *y16, const int64_t *ldy16, const int32_t *epi, float rms_eps, float head_eps,
                          void *stream);

/*
 * SwiGLU epilogue: the gate and up projections of the feed-forward block in one
 * launch whose output is already the block's hidden activation,
 *     y[b*ldy + r] = silu(g) * u,  g = sum_k Wg[r, k] x[b, k],  u = sum_k Wu[r, k] x[b, k],
 * silu(g) = g / (1 + exp(-g)), r < inter (the SwiGLU feed-forward of "Muse-
 * Glimmer-30B (text decoder) - Apple Core AI", section "The architecture, and
 * what the port had to do about it"; fusing the gate+up epilogue halves the
 * launch's output and removes the activation pass).
 * kq_repack_swiglu packs the pair so that 64-row tile t holds rows 32t..32t+31
 * of the gate matrix followed by the same rows of the up matrix:
 *   gate, up : device GGUF super-blocks, inter x cols each (alignment as kq_repack).
 *   out      : device, kq_repacked_bytes(type, 64 * ceil(inter / 32), cols) bytes,
 *              16-byte aligned; rows past inter are zero.
 * kq_gemv_swiglu then takes that buffer (w) with the same inter and cols; x, y
 * and the other arguments as kq_gemv_q4k.  Deterministic; y is within the GEMV
 * tolerance of g and u carried through silu(g) * u (see the tests).
 */
int kq_repack_swiglu(int type, int64_t inter, int64_t cols, const void *gate, const void *up, void *out,
                     void *stream);
int kq_gemv_swiglu(int type, const void *w, int64_t inter, int64_t cols, const void *x, int xtype, int64_t ldx,
                   int batch, float *y, int64_t ldy, void *ws, size_t ws_bytes, void *stream);

/*
 * Row gather: the embedding lookup of a token, the step before layer 0 of a
 * decoder whose embedding is a K-quant matrix of its own (an untied vocabulary
 * table: "Muse-Glimmer-30B (text decoder) - Apple Core AI", section "The
 * architecture, and what the port had to do about it", 202 048 rows).
 *   out[i*ldo + k] = dequant(W)[ids[i], k]   for i < n, k < cols
 *   w   : repacked weights (kq_repack with the same type, rows, cols), 16-byte aligned.
 *   ids : device, n int32 row indices, 4-byte aligned; any order, repeats allowed.
 *   out : device fp32 [n][ldo], ldo >= cols, 4-byte aligned.
 * Values are bitwise those of kq_dequant.  An id outside [0, rows) yields a row
 * of quiet NaNs (nothing outside w is read).  n = 0 enqueues nothing.
 */
int kq_gather_rows(int type, const void *w, int64_t rows, int64_t cols, const int32_t *ids, int64_t n, float *out,
                   int64_t ldo, void *stream);

/*
 * Chains: a dependent sequence of GEMV steps in ONE persistent launch.
 *
 * Every token runs the decoder's projections one after the other, each reading
 * what an earlier one produced, and its cost is the weight bytes streamed
 * ("Muse-Glimmer-30B (text decoder) - Apple Core AI", decode table and the
 * paragraph after it).  Launched one by one, each product pays a launch gap and
 * fills and drains the GPU on its own.  A chain runs all steps in one launch:
 * step j+1 issues its first weight loads while step j drains, and reads its
 * activations only after every output of step j has been written.  So x of step
 * j+1 may be y of step j (or of any earlier step): fp32 activations, with ldx
 * = ldy.  A chain runs 8-wavefront workgroups, one per CU (KQ_WG_WAVES = 4 or 8
 * sets the shape of chains and single launches alike).  Single launches use the
 * same shape above batch 1; at batch 1 they default to one 4-wavefront
 * workgroup per CU.  With the same shape the results are those of the same
 * kq_gemv_multi calls made in order (bitwise: each step runs the same
 * arithmetic in the same order); otherwise each step is within the GEMV's
 * tolerance of them.
 *
 * kq_chain_step describes one step exactly as kq_gemv_multi takes it (n = 1 for
 * a single matrix).  All steps share xtype and batch.
 *
 * Mixed weight types: the segments of one step may have different K-quant
 * types (`types`), as in the mixed-type GGUF builds (the SGLang Day-0 post's
 * GGUF checkpoints, "Q4KM" and "Q4K-Dynamic"; e.g. Q4_K q/k rows with Q6_K v
 * rows in one QKV projection).  The step still reads x once per workgroup and
 * runs in the same launch: its segments of each type form one sub-step, and
 * the sub-steps after the first run without waiting for it (they share x and
 * write other outputs).  Each sub-step's results are bitwise those of the
 * kq_gemv_fused call over its segments with the chain's workgroup shape.
 *
 * Overlap of independent steps (flags & KQ_STEP_OVERLAP): such a step does not
 * wait at the step barrier when none of its buffers (x, every y and y16, as
 * byte ranges of batch rows) meets a buffer of a step that may still be running
 * (every step since the last one that waited) in a way that orders them: its x
 * against their outputs, its outputs against their x and outputs.  It then
 * starts on the workgroups after the previous step's and runs while that step
 * drains.  Each step of such an overlapping run has a workspace region of its
 * own, so the chain's device memory grows with the run's length; a run is cut
 * by a wait once its regions would pass 512 MiB.  A step that meets such a
 * buffer waits as without the flag.  A step that skips the barrier and has
 * fewer than 8 units (64 rows x 256 columns) per CU takes one whole 64-row
 * tile per workgroup, so none of its tiles is handed over between workgroups:
 * its results are then those of its single launch planned the same way
 * (KQ_WHOLE_TILES_BELOW=8) and within the GEMV's tolerance of the default
 * plan; every other step's results are bitwise those of the same chain
 * without the flag.  This is for sequences whose steps read inputs that
 * are already in memory, such as GEMVs with activations of their own run back
 * to back; in a decoder, where each projection reads the previous one's
 * output, every step still waits.  Steps without the flag always wait.
 */
#define KQ_STEP_OVERLAP 1

typedef struct kq_chain_step {
  int32_t type;                   /* KQ_Q4_K / KQ_Q5_K / KQ_Q6_K */
  int32_t n;                      /* row segments sharing x, 1..KQ_MAX_PROJ */
  int64_t cols;                   /* K, a positive multiple of 256 */
  const void *w[KQ_MAX_PROJ];     /* device, repacked weights of each segment */
  int64_t rows[KQ_MAX_PROJ];      /* rows of each segment */
  float *y[KQ_MAX_PROJ];          /* device, fp32 outputs */
  int64_t ldy[KQ_MAX_PROJ];       /* output row strides (elements), >= rows */
  void *y16[KQ_MAX_PROJ];         /* device, optional bf16 copies of the outputs (NULL: none), as kq_gemv_fused */
  int64_t ldy16[KQ_MAX_PROJ];     /* their row strides (elements) */
  const void *x;                  /* device activations, batch rows of stride ldx */
  int64_t ldx;                    /* activation row stride (elements), >= cols */
  int32_t epilogue;               /* segment i's KQ_EPI_* code in bits 4i..4i+3 (KQ_EPI_SWIGLU: n = 1,
                                     w from kq_repack_swiglu, rows[0] = inter) */
  float rms_eps;                  /* > 0: weight-less RMSNorm of x first, as kq_gemv_fused; 0: none */
  float head_eps;                 /* epsilon of KQ_EPI_HEADNORM segments, as kq_gemv_fused */
  int32_t flags;                  /* 0 or KQ_STEP_OVERLAP (above); any other bit: KQ_ERR_SHAPE */
  int32_t types[KQ_MAX_PROJ];     /* segment i's weight type; 0 = `type` (a zeroed array: one type) */
} kq_chain_step;

typedef struct kq_chain kq_chain;

/*
 * Plan a chain of n_steps (1..65536) steps on the current device: validates
 * every step as kq_gemv_multi would, sizes the persistent grid from the
 * kernel's occupancy, and allocates the chain's device memory (the step table,
 * the step barrier's words, about 2.5 KB per step, and a workspace: the
 * largest step's size, or with KQ_STEP_OVERLAP the largest run of overlapping
 * steps' regions) and one pinned host word for its time-out flag.
 * Synchronous; must not be called inside a stream capture.  The step table is copied, so `steps` may be freed after.
 * Every x must also satisfy ((batch-1)*ldx + cols) * element size < 2^31.
 * On success *out owns the plan; release it with kq_chain_destroy.
 */
int kq_chain_create(int n_steps, const kq_chain_step *steps, int xtype, int batch, kq_chain **out);

/*
 * Enqueue one run of the chain on `stream` (one kernel launch, no allocation;
 * may be captured in a HIP graph).  Runs of one chain must not overlap in time
 * (they share its control words and workspace); different chains are
 * independent.  The device current at the call must be the chain's (else
 * KQ_ERR_DEVICE).
 *
 * Time-outs: every wait of a step for the previous one is bounded (about a
 * second; the environment variable KQ_CHAIN_SPIN, read at each run, sets the
 * poll limit).  When one gives up, the run's results are invalid: the device
 * sets the chain's error word and a pinned host word, the rest of the run's
 * waits give up at once, and any later run of the chain does nothing until
 * kq_chain_status has reset it.  kq_chain_run itself returns KQ_ERR_TIMEOUT,
 * enqueuing nothing, once the host word is set (no device synchronisation).
 */
int kq_chain_run(kq_chain *c, void *stream);

/*
 * Host only: waits[j] = 1 if step j of the chain waits at the step barrier,
 * 0 if it overlaps the steps before it (KQ_STEP_OVERLAP with independent
 * buffers; step 0 always reads 1).  n must be the chain's step count, else
 * KQ_ERR_SHAPE.
 */
int kq_chain_waits(const kq_chain *c, uint8_t *waits, int n);

/*
 * Non-synchronising: KQ_ERR_TIMEOUT if a run's wait has given up since the
 * last reset (as far as the device has progressed), else KQ_OK.
 */
int kq_chain_query(kq_chain *c);

/*
 * Synchronous: waits for the device, then returns KQ_ERR_TIMEOUT if a step's
 * wait in any run since the last call gave up, else KQ_OK.  In the first case
 * it also resets the chain (its split-tile and head counters, which a
 * workgroup that stopped waiting may have left non-zero, and both error
 * words), so the next run is valid again.
 */
int kq_chain_status(kq_chain *c);

/* Free the chain's device memory (synchronous). NULL is accepted. */
int kq_chain_destroy(kq_chain *c);

#ifdef __cplusplus
}
#endif

#endif /* KQ_H */
