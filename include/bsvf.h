/*
 * bsvf.h — C ABI of the frame-aligned block-sparse video attention library
 * (forward pass), built for AMD Instinct MI355X (gfx950).
 *
 * The operation (sources are web pages describing HeyGen's Avatar IV port to
 * TPUs; cited by page and section):
 *   - vatt-ghern.pages.dev "deep-heygen-avatar-iv-trillium-tpu", section
 *     把 block 縮到 16: block-sparse attention whose blocks are multiples of
 *     16 tokens and whose edges sit on frame edges, so no block is partly
 *     masked and no padding or mask predicate is needed.  Same point in
 *     bytechap.com "Optimizing HeyGen's Avatar IV diffusion model for Google
 *     Cloud TPUs", section How it works, and cloudcurated.com "How is HeyGen
 *     optimizing AI video on Google Cloud TPUs", Wall 2.
 *   - vatt-ghern, section 拿掉 softmax 的序列相依 (also cloudcurated Wall 3):
 *     the softmax shift of each query row may be fixed before the key loop to
 *     the Cauchy-Schwarz bound scale*|q_i|*max|k_j| computed from precomputed
 *     norms, which removes the running max and its rescaling; heads for which
 *     the bound is too loose fall back to the online running max inside the
 *     same kernel.
 *
 * Tokens are laid out frame by frame: token n belongs to frame n / T.  Query
 * frame f attends key frame g when -win_before <= g - f <= win_after, or when g
 * is one of the global frames (key side only).  Attention is bidirectional.
 *
 * Conventions for every function:
 *   - Return ATTN_OK (0) or a positive ATTN_E_* status.  On error nothing has
 *     been written and nothing launched; attn_last_error() gives a message
 *     (per calling thread).
 *   - Every buffer is owned by the caller.  The library allocates no memory
 *     and, apart from attn_fwd_noalloc's counter array (below), keeps no
 *     state of its own between calls; it never synchronizes.
 *     Device work is enqueued on the caller's stream and the call returns at
 *     once.  A device fault surfaces at the caller's next synchronization.
 *     The other state that outlives a call is the caller-given workspace
 *     attn_blocks_t.work_ctr (counters every call leaves zero).
 *   - "device" pointers are HIP device memory of the current device; "host"
 *     pointers are ordinary CPU memory.
 *   - bf16 tensors are passed as const void* to raw 16-bit bf16 storage.
 *   - Besides that array (one per GPU, shared by every attn_fwd_noalloc
 *     call on it) the library holds no global mutable state, so calls from
 *     several threads are safe as long as they share no output buffer and no
 *     work_ctr workspace, and attn_fwd_noalloc calls on one GPU do not
 *     overlap: calls that share counters must be ordered (one stream, or a
 *     stream that waits on the other's work), because each call hands out
 *     its work through those counters and resets them at its end.
 */
#ifndef BSVF_H
#define BSVF_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BSVF_ABI_VERSION 5

/* Status codes. */
enum {
  ATTN_OK = 0,
  ATTN_E_INVAL = 1,       /* NULL pointer, non-positive size, bad enum value */
  ATTN_E_ALIGN = 2,       /* not a multiple of 16 tokens, N != F*T, misaligned
                             pointer or stride, d-stride != 1 */
  ATTN_E_PATTERN = 3,     /* malformed frame pattern */
  ATTN_E_SIZE = 4,        /* output capacity too small; sizes overflow */
  ATTN_E_UNSUPPORTED = 5, /* head_dim not 64 or 128; block_q above the kernel's
                             tile; bound mode without norms */
  ATTN_E_HIP = 6          /* a HIP runtime call failed */
};

/* Softmax modes of attn_fwd. */
enum {
  ATTN_SOFTMAX_ONLINE = 0,       /* running max with rescaling, every head */
  ATTN_SOFTMAX_BOUND = 1,        /* Cauchy-Schwarz shift on eligible heads,
                                    online fallback on the rest (the method);
                                    see ATTN_PRESCALE_NATS */
  ATTN_SOFTMAX_BOUND_FORCED = 2, /* bound on every head (diagnostic only: may
                                    underflow to l = 0 on loose heads) */
  ATTN_SOFTMAX_BOUND_TILE = 3,   /* the eligibility test per query tile instead
                                    of per head: a tile takes the bound when
                                    2 * scale * max|q| over its rows * max|k|
                                    over its attended keys <= ATTN_ELIGIBLE_NATS,
                                    else the running max */
  ATTN_SOFTMAX_BOUND_EXACT = 4,  /* as ATTN_SOFTMAX_BOUND, but no head uses the
                                    prescaled Q of ATTN_PRESCALE_NATS: every
                                    bound head scales each score instead
                                    (slower, Q never rounded) */
  ATTN_SOFTMAX_BOUND_CHECKED = 5 /* as ATTN_SOFTMAX_BOUND_TILE, and a tile whose
                                    bound lies in (ATTN_ELIGIBLE_NATS,
                                    ATTN_CHECK_NATS] runs with the bound less
                                    ATTN_CHECK_SHIFT_NATS as a fixed shift
                                    (Q exact), then keeps the result iff
                                    every row's l >= 2^ATTN_CHECK_LOG2_L and
                                    nothing overflowed; else it is computed
                                    again with the running max */
};

/* Values written to head_path_out. */
enum { ATTN_PATH_ONLINE = 0, ATTN_PATH_BOUND = 1 };

/* Largest query tile attn_fwd accepts (its workgroup tile). */
#define ATTN_MAX_BLOCK_Q 256

/* Per-head eligibility limit in nats: a head takes the bound path in mode 1
 * iff 2 * scale * max_n|q_n| * max_n|k_n| <= ATTN_ELIGIBLE_NATS (inclusive).
 * This caps the gap between the fixed shift and the true row max, so the
 * largest term exp(s - m) stays far above the float32/bf16 normal range. */
#define ATTN_ELIGIBLE_NATS 60.0f

/* Eligible heads (or tiles, mode 3) whose slack bound is at most
 * ATTN_PRESCALE_NATS run with Q multiplied by scale*log2(e) and rounded to
 * bf16 once (no multiply per score); the others keep Q exact and scale each
 * score (the rounding moves a score by up to 2^-9 of scale*|q||k|, which
 * matters only for large logits).  Both use the same fixed shift. */
#define ATTN_PRESCALE_NATS 40.0f

/* ATTN_SOFTMAX_BOUND_CHECKED: tiles whose slack bound exceeds
 * ATTN_ELIGIBLE_NATS but not ATTN_CHECK_NATS run with the shift
 * m_i - ATTN_CHECK_SHIFT_NATS (m_i the bound) and check it after the fact.
 * Every term exp(s_ij - m_i') is then at most e^ATTN_CHECK_SHIFT_NATS, so l
 * and the accumulators stay finite unless |v| exceeds about e^38 / n; the
 * check tests that anyway.  Terms below the normal float32/bf16 range
 * (2^-126) are lost or denormal; over n keys they change l and the output's
 * numerator by less than n * 2^-126.  A row that keeps
 * l >= 2^ATTN_CHECK_LOG2_L therefore loses less than n * 2^-26 of it
 * (2^-12 at 16,384 keys, and only if nearly every term sits just below the
 * range).  A tile with a row outside those limits is computed again with the
 * running max; its first result is discarded, at the cost of a second pass
 * over the tile's keys. */
#define ATTN_CHECK_NATS 256.0f
#define ATTN_CHECK_LOG2_L (-100.0f)
#define ATTN_CHECK_SHIFT_NATS 40.0f

/* Frame-window pattern (host struct). */
typedef struct attn_pattern_t {
  int32_t num_frames;        /* F >= 1 */
  int32_t tokens_per_frame;  /* T: positive multiple of 16 */
  int32_t win_before;        /* >= 0: frames attended before the query frame */
  int32_t win_after;         /* >= 0: frames attended after the query frame */
  int32_t num_global;        /* >= 0 */
  const int32_t* global_frames; /* host [num_global], each in [0, F); may repeat */
} attn_pattern_t;

int attn_abi_version(void);                 /* BSVF_ABI_VERSION */
const char* attn_status_str(int status);    /* static string, never NULL */
const char* attn_last_error(void);          /* last failure on this thread */

/*
 * attn_build_blocks — host, integer only, deterministic.
 * The frame-aligned block list (vatt-ghern "deep-heygen-avatar-iv-trillium-tpu",
 * section 把 block 縮到 16: blocks are multiples of 16 tokens whose edges sit
 * on frame edges, so every block is wholly attended or absent; bytechap "How
 * it works"; cloudcurated Wall 2).
 * The block list of a pattern at query tile size block_q, canonical form:
 *   q_tiles [n_qt][2] = (first token, rows).  Frame-major; frame f is cut
 *       into T / block_q tiles of block_q rows from token f*T, then one tail
 *       tile of T % block_q rows if that is non-zero.  No tile crosses a frame.
 *   kv_ptr  [n_qt + 1] = CSR offsets of each tile's intervals in kv_iv.
 *   kv_iv   [nnz][2]  = (first key token, length): the tile's attended keys as
 *       maximal runs, ascending.  All starts and lengths are multiples of 16.
 *   *useful_pairs = number of unmasked (query, key) pairs of one head.
 * Two-call protocol: with q_tiles, kv_ptr and kv_iv all NULL, only *n_qt and
 * *nnz (and *useful_pairs if non-NULL) are written.  Otherwise all three must be
 * given and *n_qt / *nnz are read as their capacities (kv_ptr needs *n_qt + 1);
 * ATTN_E_SIZE if too small, with the needed counts written back.
 * Errors: ATTN_E_INVAL (NULL p, n_qt or nnz), ATTN_E_ALIGN (T or block_q not a
 * positive multiple of 16), ATTN_E_PATTERN (F < 1, negative window, global
 * frame out of range), ATTN_E_SIZE (F*T above INT32_MAX or capacity short).
 */
int attn_build_blocks(const attn_pattern_t* p, int32_t block_q,
                      int32_t* q_tiles, int32_t* kv_ptr, int32_t* kv_iv,
                      int64_t* useful_pairs, int32_t* n_qt, int32_t* nnz);

/*
 * attn_build_blocks_granular — host, integer only, deterministic.
 * The block list of the frame-unaware layout, for comparison with the
 * frame-aligned one (the layout the pages moved away from: fixed blocks
 * whose edges ignore frame edges, so some blocks are partly masked; vatt-ghern
 * section 把 block 縮到 16, bytechap "How it works", cloudcurated Wall 2).
 *   q_tiles [n_qt][2]: tiles of block_q consecutive rows from token 0 (the last
 *       one shorter when N % block_q != 0), regardless of frames.
 *   kv_iv [nnz][2], kv_ptr: per tile, maximal ascending runs of key blocks of
 *       `granule` consecutive keys (the last block of the sequence shorter)
 *       that some (row, key) pair of the tile attends, split where the flag
 *       changes;
 *   kv_flag [nnz]: 1 when some pair of the run's blocks is masked (the kernel
 *       then evaluates the frame mask per element), 0 when every pair is
 *       attended.
 *   *useful_pairs: as attn_build_blocks.
 * granule must be a positive multiple of 64 (so every 64-key stage lies in
 * one run), block_q a positive multiple of 16.  Same two-call protocol as
 * attn_build_blocks (kv_flag joins the three arrays: all NULL or none).
 * Errors: as attn_build_blocks; ATTN_E_ALIGN also for a bad granule.
 */
int attn_build_blocks_granular(const attn_pattern_t* p, int32_t granule, int32_t block_q,
                               int32_t* q_tiles, int32_t* kv_ptr, int32_t* kv_iv,
                               int32_t* kv_flag, int64_t* useful_pairs, int32_t* n_qt,
                               int32_t* nnz);

/*
 * attn_build_schedule — host, integer only, deterministic.
 * Launch order for attn_fwd over batch*heads*n_qt work items (item
 * w = tile + n_qt * (head + heads * batch_index)).  A tile's cost is
 * keys * max(rows, R/2), R the largest tile's rows, or keys * R/3 for a short
 * tile (at most R/4 rows).  Workgroup i runs on
 * accelerator die i % num_xcd and takes the next item of that die's queue:
 *   group > 0: items by decreasing cost (ties keep the natural order), cut
 *     into groups of `group` consecutive items, group j appended to die
 *     j % num_xcd;
 *   group == 0: the tiles of one (batch, head) that share their key
 *     intervals (one query frame's tiles) form a set that stays together on
 *     one die, so they stream the same K and V through that die's L2.  The
 *     sets, in (batch, head, frame) order, are cut into num_xcd contiguous
 *     runs of about equal cost (a set goes to the die whose share of the
 *     total cost holds the middle of the set's cost), so neighbouring frames,
 *     which share most of their keys, run on one die.  Short tiles are left
 *     out of their sets and follow all of their die's sets, in the same
 *     order.
 * Queues are padded with -1 to a common depth (a multiple of `group` when
 * group > 0); such a workgroup exits at once.  The result is a permutation of
 * all items plus padding; it changes only the execution order, never results.
 * Inputs are the host block list from attn_build_blocks.  Two-call protocol:
 * with work_order NULL only *n_work is written; otherwise *n_work is the
 * capacity (ATTN_E_SIZE if short, needed count written back).
 * Errors: ATTN_E_INVAL (NULL arrays, non-positive sizes, group < 0,
 * num_xcd < 1), ATTN_E_SIZE.
 */
int attn_build_schedule(const int32_t* q_tiles, const int32_t* kv_ptr,
                        const int32_t* kv_iv, int32_t n_qt, int32_t batch,
                        int32_t heads, int32_t group, int32_t num_xcd,
                        int32_t* work_order, int32_t* n_work);

/*
 * attn_norms — device, fp32 results, HBM-bound (reads Q and K once).
 * The precomputed norms the bound softmax needs (vatt-ghern, section
 * 拿掉 softmax 的序列相依):
 *   q_norm  [B][H][N]     |q_n|_2
 *   k_gmax  [B][H][N/16]  max |k_n|_2 over each 16-key granule
 *   head_max[B][H][2]     (max_n |q_n|_2, max_n |k_n|_2)
 * Outputs are contiguous fp32 device buffers.  Sums of squares accumulate in
 * fp32.  q, k: device bf16 [B][H][N][D] addressed through element strides
 * {b, h, n} (d-stride 1); the default contiguous layout is
 * {H*N*D, N*D, D}, and [B][N][H][D] is {N*H*D, D, H*D}.
 * Errors: ATTN_E_INVAL (NULL, non-positive sizes), ATTN_E_ALIGN (N % 16,
 * pointer not 16-byte aligned, stride not a multiple of 8), ATTN_E_UNSUPPORTED
 * (D not 64 or 128), ATTN_E_HIP (launch failed).
 */
int attn_norms(const void* q, const void* k, int32_t batch, int32_t heads,
               int32_t seq_len, int32_t head_dim, const int64_t* q_strides,
               const int64_t* k_strides, float* q_norm, float* k_gmax,
               float* head_max, hipStream_t stream);

/* Device block list for attn_fwd (pointers to device copies of the host
 * arrays from attn_build_blocks / attn_build_schedule). */
typedef struct attn_blocks_t {
  const int32_t* q_tiles;    /* device [n_qt][2] */
  const int32_t* kv_ptr;     /* device [n_qt + 1] */
  const int32_t* kv_iv;      /* device [nnz][2] */
  int32_t n_qt;
  int32_t nnz;
  int32_t block_q;           /* tile size the list was built with, <= ATTN_MAX_BLOCK_Q */
  const int32_t* work_order; /* device [n_work] from attn_build_schedule, or NULL
                                for the natural order (one workgroup per item) */
  int32_t n_work;
  int32_t num_xcd;           /* the num_xcd work_order was built with (1..32);
                                read only when work_ctr is not NULL */
  int32_t* work_ctr;         /* device int32 [num_xcd + 1] workspace, or NULL.
                                Given (with a work_order), one launch runs
                                every item on its own path (bound or online),
                                one workgroup per CU, each taking items from its
                                accelerator die's queue of work_order and then
                                from the others', counting handed-out slots
                                here: dies that run faster take over the slower
                                ones' work, and online items share the CUs with
                                bound ones.  (In mode 1 the launch is two
                                kernels in a row on the stream: one holding
                                both loops and one holding the online loop
                                alone, with its own register allocation; each
                                first tests the head norms on the device, and
                                only the second takes items when no head
                                passes with the prescaled Q, only the first
                                otherwise.)  The caller zeroes it once before its
                                first use; every call leaves it zero again.
                                Calls that share it must not overlap (one
                                stream, or a stream that waits for the other
                                stream's call); overlapping calls would split
                                each other's items and leave outputs partly
                                unwritten, undetected.  NULL: one
                                workgroup per item, in work_order's fixed
                                order. */
} attn_blocks_t;

/*
 * attn_fwd — device: the block-sparse attention forward pass over the
 * frame-aligned block list (vatt-ghern "deep-heygen-avatar-iv-trillium-tpu",
 * section 把 block 縮到 16), with either the online running-max softmax or
 * the Cauchy-Schwarz shift fixed before the key loop from precomputed norms
 * and a per-head fallback to the running max (same page, section
 * 拿掉 softmax 的序列相依; cloudcurated Wall 3).
 *   O[b,h,i,:] = sum_j P_ij v_j,  P_ij = exp(s_ij - m_i) / l_i over the keys j
 *   the tile of row i attends, s_ij = scale * <q_i, k_j>,
 *   LSE[b,h,i] = m_i + ln l_i  (natural log).
 * bf16 MFMA products with fp32 accumulation; P is rounded to bf16 for the
 * P*V product; O is rounded to bf16 (nearest even); LSE is fp32.
 *   q, k, v: device bf16 [B][H][N][D] via strides; o: device bf16 output.
 *   strides: host int64 [4][3], element strides {b, h, n} of q, k, v, o
 *       (d-stride 1 for all four).
 *   lse: device fp32 [B][H][N] contiguous, or NULL.
 *   shift_out: device fp32 [B][H][N] or NULL; receives the shift m_i used by
 *       the row (natural-log units; the bound itself on bound heads, the
 *       bound less ATTN_CHECK_SHIFT_NATS on tiles kept by the check).
 *   scale: softmax scale (usually 1/sqrt(D)); must be > 0 and finite.
 *   blocks: block list (see attn_blocks_t).  It must come from
 *       attn_build_blocks for this N; the kernel skips any tile or interval
 *       that lies outside [0, N) or exceeds block_q, so a corrupt list cannot
 *       make it read or write out of bounds, but rows it skips are not written.
 *   q_norm, k_gmax, head_max: attn_norms outputs; needed when softmax_mode is
 *       not ATTN_SOFTMAX_ONLINE, ignored (may be NULL) otherwise.
 *   softmax_mode: ATTN_SOFTMAX_*.  The bound shift is
 *       m_i = scale * |q_i| * max{k_gmax over the tile's intervals} * (1 + 2^-8);
 *       the factor keeps it above every score the kernel computes (fp32 dot
 *       products and norms).  Heads (tiles, mode 3) whose slack bound is at
 *       most ATTN_PRESCALE_NATS (except in mode 4), and every head in mode 2,
 *       use Q multiplied by scale*log2(e) and rounded to bf16 once; the rest
 *       use Q as given.  In mode 5 a tile that fails its check is computed
 *       twice, and its outputs are those of the second (running max) pass.
 *   head_path_out: device int32 [B][H] or NULL; receives ATTN_PATH_* per head
 *       (for ATTN_SOFTMAX_BOUND_TILE and _CHECKED: the path of the head's
 *       first tile, after its check).
 * Errors: ATTN_E_INVAL (NULL tensor or block pointers, non-positive sizes,
 * bad mode, bad scale), ATTN_E_ALIGN (N % 16, block_q % 16, misaligned pointer
 * or stride), ATTN_E_UNSUPPORTED (D not 64/128, block_q > ATTN_MAX_BLOCK_Q,
 * bound mode with NULL norms), ATTN_E_SIZE (a head's span exceeds 2^31
 * elements), ATTN_E_HIP (launch failed).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             float* shift_out, int32_t batch, int32_t heads, int32_t seq_len,
             int32_t head_dim, const int64_t* strides, float scale,
             const attn_blocks_t* blocks, const float* q_norm,
             const float* k_gmax, const float* head_max, int32_t softmax_mode,
             int32_t* head_path_out, hipStream_t stream);

/* Largest num_xcd attn_fwd_noalloc accepts (its counter array holds
 * ATTN_NOALLOC_MAX_XCD + 1 int32). */
#define ATTN_NOALLOC_MAX_XCD 32

/*
 * attn_fwd_noalloc — device; attn_fwd for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Same arguments, results
 * and errors as attn_fwd, with these differences:
 *   - blocks->work_ctr must be NULL: the persistent launch's slot counters
 *     live in a fixed array of the library (ATTN_NOALLOC_MAX_XCD + 1 int32 in
 *     device memory, one copy per GPU, held until the process ends), which
 *     each call clears with a one-workgroup kernel on `stream` before its
 *     launch;
 *   - blocks->work_order is required (the persistent launch's queues), and
 *     blocks->num_xcd must be in [1, ATTN_NOALLOC_MAX_XCD]: ATTN_E_SIZE above
 *     it, ATTN_E_INVAL for NULL work_order, a non-NULL work_ctr, num_xcd < 1 or
 *     n_work not a multiple of num_xcd;
 *   - the call allocates nothing (no hipMalloc, hipFree or allocating library
 *     routine).  Its first call on a device looks the array up there
 *     (hipGetSymbolAddress); ATTN_E_HIP if that fails, ATTN_E_UNSUPPORTED for
 *     a device index above 63.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (several streams, or several threads) race and may leave outputs partly
 * unwritten.  Order them (one stream, or events).
 */
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                     float* shift_out, int32_t batch, int32_t heads, int32_t seq_len,
                     int32_t head_dim, const int64_t* strides, float scale,
                     const attn_blocks_t* blocks, const float* q_norm,
                     const float* k_gmax, const float* head_max, int32_t softmax_mode,
                     int32_t* head_path_out, hipStream_t stream);

/*
 * attn_fwd_masked — device; attn_fwd over the frame-unaware layout of
 * attn_build_blocks_granular, for comparison with the frame-aligned kernel
 * (the pages' point: blocks that ignore frame edges need a mask predicate on
 * every partly attended block; vatt-ghern section 把 block 縮到 16, bytechap
 * "How it works").  Same arguments, results and errors as attn_fwd, plus:
 *   kv_flag  device int32 [blocks->nnz]: the flags from
 *            attn_build_blocks_granular (1 = evaluate the frame mask per
 *            score; 0 = every pair attended);
 *   pattern  host: the frame pattern the list was built from (its
 *            num_frames * tokens_per_frame must equal seq_len).
 * The result is the same attention as attn_fwd on the aligned list, up to
 * summation order.  Requires tokens_per_frame >= 64, global frames below 64,
 * and a list built with a granule that is a multiple of 64 (each 64-key stage
 * then lies in one run); ATTN_E_UNSUPPORTED / ATTN_E_PATTERN otherwise.
 * Softmax modes 0 to 4 (ATTN_SOFTMAX_BOUND_CHECKED: ATTN_E_UNSUPPORTED).
 */
int attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse,
                    float* shift_out, int32_t batch, int32_t heads, int32_t seq_len,
                    int32_t head_dim, const int64_t* strides, float scale,
                    const attn_blocks_t* blocks, const int32_t* kv_flag,
                    const attn_pattern_t* pattern, const float* q_norm, const float* k_gmax,
                    const float* head_max, int32_t softmax_mode, int32_t* head_path_out,
                    hipStream_t stream);

/*
 * attn_qk_prep — device, HBM-bound: the producer of Q and K with the norms of
 * attn_norms in its epilogue.  The pages hand the attention kernel
 * precomputed norms (vatt-ghern, section 拿掉 softmax 的序列相依) and fuse
 * producer stages so that each writes what the next reads, in its layout
 * (cloudcurated, layout contracts after Wall 3).  Per row x of one head
 * (fp32 arithmetic, one rounding to bf16, nearest even):
 *   y   = x * gamma / sqrt(mean_e x_e^2 + eps)              (QK RMS norm)
 *   out_2i   = y_2i * cos[n][i] - y_2i+1 * sin[n][i]        (rotary pairs)
 *   out_2i+1 = y_2i * sin[n][i] + y_2i+1 * cos[n][i]
 * then, over the rounded rows just written: q_norm, k_gmax and head_max
 * exactly as attn_norms defines them, so attn_fwd can take them directly.
 *   q_in, k_in: device bf16 [B][H][N][D]; q_out, k_out: device bf16 outputs
 *       (an output may be its own input with identical strides; q_out and
 *       k_out must not alias each other or the other input; any other
 *       overlap between outputs and inputs is undefined and not detected).
 *   strides: host int64 [4][3], element strides {b, h, n} of q_in, k_in,
 *       q_out, k_out (d-stride 1), so e.g. a [B][N][H][D] projection output
 *       is read in place and written in the attention's [B][H][N][D].
 *   q_gamma, k_gamma: device fp32 [D] RMS-norm weights (one per tensor,
 *       shared by the heads).  eps: finite, >= 0.
 *   rope_cos, rope_sin: device fp32 [N][D/2] contiguous; entry [n][i] turns
 *       pair (2i, 2i+1) of token n (any 1-D or 3-D position scheme; the
 *       identity is cos = 1, sin = 0).
 *   q_norm, k_gmax, head_max: attn_norms' outputs (contiguous fp32), all
 *       three or all NULL (then only Q and K are written).
 * Pointers 16-byte aligned.  Caller owns every buffer; enqueued on `stream`.
 * Errors: ATTN_E_INVAL (NULL, non-positive sizes, bad eps, forbidden
 * aliasing, only some norm outputs), ATTN_E_ALIGN (N % 16, misaligned
 * pointer or stride), ATTN_E_UNSUPPORTED (D not 64 or 128), ATTN_E_SIZE
 * (B * H > 65535 or too many rows), ATTN_E_HIP (launch failed).
 * All checks run before any launch; on error nothing is written.
 */
int attn_qk_prep(const void* q_in, const void* k_in, void* q_out, void* k_out,
                 int32_t batch, int32_t heads, int32_t seq_len, int32_t head_dim,
                 const int64_t* strides, const float* q_gamma, const float* k_gamma,
                 float eps, const float* rope_cos, const float* rope_sin,
                 float* q_norm, float* k_gmax, float* head_max, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BSVF_H */
