/*
 * lora_proj.h — the mixed-adapter LoRA projection on AMD MI355X (gfx950).
 *
 * What it computes ("two 27B models on a single RTX 5090", section 3 weights
 * figure and section 4 request-path figure): each changed matrix of the adapted
 * model equals the base matrix plus a rank-r product B.A, and a request that
 * names the adapter runs the base product plus the adapter's two thin matrices,
 * while requests that name the base model use the base weights alone, in the
 * same batch.  With s the call's scale (1.0 reproduces the unscaled merge):
 *
 *     Y[m,:] = X[m,:] W^T + s (X[m,:] A_a^T) B_a^T   rows of a segment naming adapter a
 *     Y[m,:] = X[m,:] W^T                            rows of base-only segments
 *
 * Layout.  Every matrix is dense and row-major with the reduction index
 * contiguous (the nn.Linear weight layout): X is M x K, W is N x K, A_a is
 * r x K, B_a is N x r, Y is M x N.  Rows are packed (leading dimension = row
 * length).  Device pointers must be 16-byte aligned.
 *
 * Segments.  The rows of one request are contiguous.  Segment g covers rows
 * [seg_starts[g], seg_starts[g+1]); seg_adapter[g] is -1 (base-only) or an
 * adapter index in [0, n_adapters).  seg_starts[0] == 0, entries never
 * decrease, seg_starts[n_seg] == M.  Empty segments are allowed.
 *
 * Precision.  LORA_BF16: bf16 inputs and output, fp32 accumulation, the
 * intermediate X A^T held at fp32-equivalent precision, one round-to-nearest-
 * even to bf16 at the store.  LORA_BF16_F32OUT: the same kernels with an fp32
 * store.  LORA_F32: fp32 inputs and output (test mode, not tuned for speed).
 *
 * Streams and ownership.  Calls are asynchronous on `stream` and return once
 * the work is enqueued.  The caller owns every buffer: device buffers must stay
 * valid until the stream work completes; host arrays (seg_starts, seg_adapter,
 * A, B) may be released as soon as the call returns.  The library allocates no
 * memory per call and keeps no state between calls; it never prints, aborts or
 * falls back to another path.  Concurrent calls need separate workspaces and
 * outputs.
 *
 * Errors.  Every argument is checked on the host before anything is launched;
 * on error the call returns the code, launches nothing and leaves Y untouched.
 * A failed launch returns LORA_EHIP; faults during execution surface at the
 * caller's next synchronisation.  M == 0 is a successful no-op.
 */
#ifndef LORA_PROJ_H
#define LORA_PROJ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lora_status {
  LORA_OK = 0,
  LORA_EINVAL = 1,        /* null pointer, negative or inconsistent size, misalignment, Y overlapping an input */
  LORA_ESEGMENTS = 2,     /* segment table malformed */
  LORA_EADAPTER = 3,      /* adapter index out of range, or its A/B pointer is null */
  LORA_EUNSUPPORTED = 4,  /* shape, rank, dtype or table size outside the documented limits */
  LORA_EWORKSPACE = 5,    /* workspace missing or smaller than lora_proj_workspace_bytes() */
  LORA_EHIP = 6,          /* the HIP runtime reported an error while enqueueing */
  LORA_EHANDOVER = 7      /* lora_workspace_status: a decode call on the workspace lost a hand-over */
} lora_status;

typedef enum lora_dtype {
  LORA_BF16 = 0,          /* bf16 X, W, A, B and Y */
  LORA_F32 = 1,           /* fp32 X, W, A, B and Y (test mode) */
  LORA_BF16_F32OUT = 2    /* bf16 X, W, A, B; fp32 Y */
} lora_dtype;

/* Documented limits (checked; anything beyond returns LORA_EUNSUPPORTED):
 *   - at most LORA_MAX_SEGMENTS segments once empty segments are dropped and neighbours
 *     naming the same adapter are merged;
 *   - n_adapters <= LORA_MAX_ADAPTERS;
 *   - rank a multiple of 16 in [LORA_MIN_RANK, LORA_MAX_RANK] when any row names an adapter;
 *   - K a multiple of 8;
 *   - every operand (X, W, each A_a and B_a, Y, the used workspace) smaller than 2 GiB. */
#define LORA_MAX_SEGMENTS 256
#define LORA_MAX_ADAPTERS 32
#define LORA_MIN_RANK 16
#define LORA_MAX_RANK 512
/* Sliced calls (lora_proj_sliced): at most LORA_MAX_SLICES slices, each of a
 * width that is a multiple of LORA_SLICE_ALIGN output columns. */
#define LORA_MAX_SLICES 4
#define LORA_SLICE_ALIGN 256
/* Bytes at the start of every workspace reserved for the decode path's
 * counters (see lora_proj's `workspace`). */
#define LORA_WORKSPACE_COUNTER_BYTES 65536

/*
 * lora_proj — one projection call over a batch of rows from several requests.
 *
 *   X            device, M x K (dtype's input type)
 *   seg_starts   HOST, n_seg + 1 int32
 *   seg_adapter  HOST, n_seg int32, -1 or 0 .. n_adapters-1
 *   n_seg        number of segments (>= 1 when M > 0)
 *   W            device, N x K
 *   A            HOST array of n_adapters device pointers, each r x K (entries may be
 *                NULL for adapters no non-empty segment names)
 *   B            HOST array of n_adapters device pointers, each N x r
 *   n_adapters   0 .. LORA_MAX_ADAPTERS
 *   rank         r, shared by all adapters of the call (ignored when no row names an adapter)
 *   scale        s, applied to the adapter term of every adapter row
 *   Y            device, M x N, fully overwritten; must not overlap X, W, any A/B or the workspace
 *   workspace    device scratch of at least lora_proj_workspace_bytes(M, N, K, rank,
 *                n_adapters, dtype) bytes (may be NULL with size 0 when that is 0).  Its
 *                first LORA_WORKSPACE_COUNTER_BYTES are a counter area that the blocks of
 *                one decode launch (at most 128 rows) use to hand work to each other.  The
 *                area must be zero when the workspace is first used (allocate it
 *                zero-filled); every call that counts on a counter puts it back to zero, so
 *                it needs no clearing between calls.  Counts left behind by a call that
 *                never finished make later calls on the workspace wrong: where an arrival
 *                finds a count past its total, the kernel stores NaN over the outputs it
 *                owns and sets a sticky error bit in the area's last 8 bytes, which
 *                lora_workspace_status reports before it restores the whole area.
 *                The rest is scratch whose contents are not preserved.  Calls that share
 *                a workspace must not overlap in time (order them on one stream)
 *   stream       HIP stream the work is ordered on (0 = the null stream)
 */
lora_status lora_proj(const void* X,
                      const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                      const void* W,
                      const void* const* A, const void* const* B,
                      int32_t n_adapters, int32_t rank, float scale,
                      void* Y,
                      int64_t M, int64_t N, int64_t K,
                      lora_dtype dtype,
                      void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * lora_proj_ex — lora_proj with two optional timing events.
 *
 * Identical arguments, checks and results; in addition, when main_start or
 * main_stop is not NULL it is recorded on `stream` at the start / end of the
 * call's dominant work, so that it can be timed on its own: for batches of
 * more than 128 rows, the output kernel (base product with the adapter expand
 * and the store; the shrink before it is excluded); for smaller batches, the
 * call's single kernel.
 * The events belong to the caller and must have been created on the current
 * device.
 */
lora_status lora_proj_ex(const void* X,
                         const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                         const void* W,
                         const void* const* A, const void* const* B,
                         int32_t n_adapters, int32_t rank, float scale,
                         void* Y,
                         int64_t M, int64_t N, int64_t K,
                         lora_dtype dtype,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream,
                         hipEvent_t main_start, hipEvent_t main_stop);

/*
 * lora_proj_multi — lora_proj with one scale per adapter.
 *
 * Several adapters serve one batch ("two 27B models on a single RTX 5090",
 * section 4 request-path figure: each request names its model, and requests
 * naming different models share the batch).  Rows of a segment naming adapter
 * a get
 *
 *     Y[m,:] = X[m,:] W^T + scales[a] (X[m,:] A_a^T) B_a^T
 *
 * and base-only rows get X[m,:] W^T, exactly as in lora_proj.  Arguments,
 * checks, workspace and results are lora_proj's, with
 *
 *   scales       HOST array of n_adapters floats (may be released on return);
 *                NULL with n_adapters > 0 returns LORA_EINVAL
 *
 * in place of the single `scale`.  All adapters of one call share `rank`;
 * lora_proj_ranked takes adapters of different ranks, each stored compact.
 */
lora_status lora_proj_multi(const void* X,
                            const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                            const void* W,
                            const void* const* A, const void* const* B,
                            int32_t n_adapters, int32_t rank, const float* scales,
                            void* Y,
                            int64_t M, int64_t N, int64_t K,
                            lora_dtype dtype,
                            void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * lora_proj_sliced — several projections of the same rows in one call.
 *
 * Projections that read the same X (the query, key and value matrices of a
 * layer, or its gate and up matrices) are served as one matrix whose W is the
 * concatenation of the slices' weights along N, the way the pages' server
 * stores such groups (section 4 request-path figure: each changed matrix runs
 * the base product plus the adapter's two thin matrices; a merged group runs
 * that for every member).  With S = n_slices and slice s covering output
 * columns [c_s, c_s + slice_n[s]), each adapter a brings its slices' factors
 * stacked:
 *
 *   A[a]   device, (S r) x K: rows s r .. s r + r - 1 are slice s's A_{a,s}
 *   B[a]   device, N x r: rows c_s .. c_s + slice_n[s] - 1 are slice s's B_{a,s}
 *
 * and rows of a segment naming adapter a get, on the columns of slice s,
 *
 *     Y[m, cols_s] = X[m,:] W[cols_s,:]^T + scales[a] (X[m,:] A_{a,s}^T) B_{a,s}^T
 *
 * which is exactly S separate lora_proj_multi calls, one per slice, with their
 * outputs side by side.  Base-only rows get X[m,:] W^T.
 *
 *   n_slices     1 .. LORA_MAX_SLICES (1 is lora_proj_multi)
 *   slice_n      HOST, n_slices int64: each a positive multiple of LORA_SLICE_ALIGN
 *                when n_slices > 1, summing to N (else LORA_EUNSUPPORTED / LORA_EINVAL)
 *   scales       HOST, n_adapters floats; NULL with n_adapters > 0 is LORA_EINVAL
 *   workspace    at least lora_proj_sliced_workspace_bytes(M, N, K, rank, n_slices,
 *                n_adapters, dtype) bytes, with lora_proj's counter-area contract
 *
 * Every other argument, check and guarantee is lora_proj's.  The shared
 * intermediate X A_a^T is S r wide, so it is computed once for all slices.
 */
lora_status lora_proj_sliced(const void* X,
                             const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                             const void* W,
                             const void* const* A, const void* const* B,
                             int32_t n_adapters, int32_t rank, const float* scales,
                             int32_t n_slices, const int64_t* slice_n,
                             void* Y,
                             int64_t M, int64_t N, int64_t K,
                             lora_dtype dtype,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * lora_proj_ranked — lora_proj_sliced with each adapter at its own rank.
 *
 * Adapter a has rank ranks[a] (each 16 .. 512 and a multiple of 16, else
 * LORA_EUNSUPPORTED): A[a] is (n_slices x ranks[a]) x K, slice s taking rows
 * s ranks[a] .. (s + 1) ranks[a] - 1, and B[a] is N x ranks[a], both stored
 * compact.  Each row gets its own adapter's term at that adapter's rank: an
 * adapter of rank 64 beside one of rank 256 reads and multiplies 64-wide
 * factors, not zero-padded 256-wide ones ("two 27B models on a single RTX 5090",
 * section 4: every request is served with its own adapter).  The result equals
 * lora_proj_sliced with every adapter zero-padded to the largest rank.
 *
 *   ranks        HOST, n_adapters int32 (entries of adapters no row names are ignored)
 *   scales       HOST, n_adapters floats
 *   workspace    at least lora_proj_sliced_workspace_bytes(M, N, K, r_max, n_slices,
 *                n_adapters, dtype), r_max the largest rank of an adapter a row names
 *
 * Everything else, including the checks and errors, is lora_proj_sliced's;
 * ranks or scales NULL with n_adapters > 0 is LORA_EINVAL.
 */
lora_status lora_proj_ranked(const void* X,
                             const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                             const void* W,
                             const void* const* A, const void* const* B,
                             int32_t n_adapters, const int32_t* ranks, const float* scales,
                             int32_t n_slices, const int64_t* slice_n,
                             void* Y,
                             int64_t M, int64_t N, int64_t K,
                             lora_dtype dtype,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Workspace bytes lora_proj_sliced needs (an upper bound over segment tables naming at most
 * n_adapters adapters, counter area included; 0 for invalid arguments).  With n_slices == 1
 * it equals lora_proj_workspace_bytes. */
size_t lora_proj_sliced_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t rank, int32_t n_slices,
                                        int32_t n_adapters, lora_dtype dtype);

/*
 * lora_proj_q4 — the sliced call with the base weights in 4-bit form.
 *
 * "two 27B models on a single RTX 5090", section 4 memory figure: the card
 * serves a 4-bit copy of the base weights beside the bf16 adapter.  The pages
 * print no format; this one is W4A16 with groups of 128 along K (AutoRound's
 * default layout):
 *
 *   Wq       device, N x K/2 bytes: the 4-bit codes q (0..15) of row n, two per
 *            byte along K; code k sits in byte k/2, low nibble for even k, high
 *            nibble for odd k
 *   Wp       device, (K/128) x N uint32 params words: word [g][n] holds the bf16
 *            scale s (bits 0-15) and the zero point z (bits 16-23) of the group of
 *            k in [128 g, 128 g + 128) of row n
 *
 * and the base weight is W[n][k] = s (q - z).  The result is lora_proj_sliced's
 * with that W.  The kernels round each dequantized weight to bf16 (nearest,
 * ties to even) before it meets the bf16 activations, an error of at most half
 * a bf16 ulp of the weight.  Batches of at most 128 rows read the codes
 * straight from HBM (a quarter of the bf16 bytes); larger batches first expand
 * them into a bf16 copy in the workspace, since those calls are bound by the
 * matrix units, not by memory.
 *
 * Extra limits: K a multiple of 128; dtype LORA_BF16 or LORA_BF16_F32OUT (the
 * fp32 test mode is not offered, LORA_EUNSUPPORTED).  Wp must not be NULL
 * (LORA_EINVAL).  workspace: at least lora_proj_q4_workspace_bytes(...) bytes.
 */
lora_status lora_proj_q4(const void* X,
                         const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                         const void* Wq, const void* Wp,
                         const void* const* A, const void* const* B,
                         int32_t n_adapters, int32_t rank, const float* scales,
                         int32_t n_slices, const int64_t* slice_n,
                         void* Y,
                         int64_t M, int64_t N, int64_t K,
                         lora_dtype dtype,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Workspace bytes of lora_proj_q4 (0 for invalid arguments).  For more than 128 rows it
 * includes the bf16 copy of W (N K 2 bytes). */
size_t lora_proj_q4_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t rank, int32_t n_slices,
                                    int32_t n_adapters, lora_dtype dtype);

/* Workspace bytes lora_proj needs for any segment table of this shape that names at most
 * n_adapters adapters (an upper bound), counter area included.  Returns 0 for invalid
 * arguments.  Batches of at most 128 rows (the decode path) always need a workspace, for its
 * counters and split-K partial sums; larger batches need one only when some row names an
 * adapter: the counter area, s X A^T (M x n_slices rank, 4 bytes an element) and, when the
 * grid of 128 x 128 tiles of s X A^T is small (at most 128 tiles, ceil(M/128) x
 * ceil(n_slices rank / 128)) and K long enough to give each split at least 8 steps of 64
 * (K > 960), fp32 partial sums of that product split over K (64 KiB per tile and split, at
 * most 8 splits). */
size_t lora_proj_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t rank, int32_t n_adapters,
                                 lora_dtype dtype);

/* Name of the kernel path lora_proj takes for this shape: "prefill" (more than 128 rows),
 * "decode" (at most 128 rows) or "f32" (test mode)
 * ("invalid" for arguments lora_proj would reject).  A pure function of its arguments. */
const char* lora_proj_path(int64_t M, int64_t N, int64_t K, int32_t rank, lora_dtype dtype);

/* Activation rows per output tile of the prefill output kernel for this shape: 256, 192 or 128
 * (the tile is always 256 output columns wide).  The kernel runs one tile per CU in whole waves
 * over the 256 CUs, so a batch of 2,054 rows, 9 tiles of 256 rows by 20 column tiles (0.70 of a
 * wave), takes 11 tiles of 192 rows instead (one wave of shorter tiles).  0 where lora_proj does
 * not take the prefill path (at most 128 rows, the f32 test mode) or would reject the arguments.
 * A pure function of its arguments. */
int32_t lora_proj_tile_rows(int64_t M, int64_t N, int64_t K, lora_dtype dtype);

/*
 * lora_proj_noalloc — lora_proj for callers that cannot allocate memory.
 *
 * For code under HIP graph capture, tight serving loops, or harnesses that forbid
 * hipMalloc.  Arguments, checks and results are lora_proj's, without the
 * workspace pair: the call's scratch (the decode path's counters, partial sums
 * and T; the prefill path's T) lives in a fixed device array of
 * LORA_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held from the
 * first call on that GPU until the process ends.  The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine); the caller still passes X,
 * W, A, B and Y.
 *
 *   - A call whose scratch would exceed LORA_NOALLOC_SCRATCH_BYTES (see
 *     lora_proj_workspace_bytes) returns LORA_EWORKSPACE and launches nothing.
 *     At 64 MiB this covers every shape above at rank 256 up to 32,768 rows of
 *     T (prefill) and every decode batch of up to 128 rows.
 *   - Decode calls (at most 128 rows) first clear the array's counter area with
 *     a small kernel on `stream`, so a call never depends on what an earlier one
 *     left there.  A lost hand-over still gives NaN outputs (there is no status
 *     query for the array).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in
 *     time on one GPU (different streams, threads or processes' contexts on the
 *     same device) race and give wrong results.  Order them on one stream.
 *   - The first call on a GPU looks up the array's device address (it must run
 *     with that device current); a runtime failure there returns LORA_EHIP.
 */
#define LORA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
lora_status lora_proj_noalloc(const void* X,
                              const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                              const void* W,
                              const void* const* A, const void* const* B,
                              int32_t n_adapters, int32_t rank, float scale,
                              void* Y,
                              int64_t M, int64_t N, int64_t K,
                              lora_dtype dtype,
                              hipStream_t stream);

/* Static description of a status code; never NULL. */
const char* lora_status_string(lora_status s);

/*
 * lora_workspace_status — did a decode call on this workspace lose a hand-over?
 *
 * A decode launch (at most 128 rows) hands T = s X A^T from the blocks that
 * compute it to the blocks that add it, and K-part sums between blocks, through
 * counters in the workspace's counter area.  Waiting is bounded: if a block gives
 * up waiting for T (other work held the GPU's compute units for about 0.3 s), or a
 * count goes past its expected total, the kernel sets a sticky bit in the last 8
 * bytes of the counter area, stores NaN in place of the output columns that
 * depended on the hand-over, and exits.  The pages' own lesson is that a silent
 * slow or wrong path is the failure to avoid ("serving-qwen3-8-27b-on-one-
 * rtx-3090", Installing: a missing header made the server slower with nothing in
 * its logs); this call is how the caller sees it.
 *
 *   workspace        device, a workspace passed to earlier calls (16-byte aligned)
 *   workspace_bytes  its size, at least LORA_WORKSPACE_COUNTER_BYTES
 *   stream           the stream those calls were ordered on
 *
 * Synchronizes `stream`, reads the bits, and clears them (a one-word kernel on
 * `stream`, then a second synchronization).  Returns LORA_OK when no call since the
 * last query lost a hand-over, LORA_EHANDOVER when one did, LORA_EINVAL for a bad
 * argument and LORA_EHIP for a runtime error.
 */
lora_status lora_workspace_status(void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * lora_debug_handover_fault — test hook for the failure path above.
 *
 * While `on` is non-zero, every decode call with adapter rows that is enqueued
 * afterwards waits for one T group more than exists, with a short bounded spin,
 * so its waits give up at once: the call's error bit is set and its output
 * columns hold NaN, and every block still exits normally.  Process-wide; for
 * tests only.  Returns the previous setting.
 */
int32_t lora_debug_handover_fault(int32_t on);

/*
 * lora_decode_plan_describe — the launch plan a decode call (1 .. 128 rows) of this
 * shape would use, for inspection and host-side tests; nothing is launched.
 *
 *   M, N, K, rank, n_slices, slice_n   as in lora_proj_sliced (slice_n may be NULL
 *                                      when n_slices == 1)
 *   n_used                             adapters the batch's rows name (0 .. LORA_MAX_ADAPTERS)
 *   out                                HOST, receives up to n_out values, in order:
 *     MT                16-row activation tiles (2, 4, 5 or 8)
 *     nst, nrs          64-wide K units per weight tile; 64-wide rank units per expand half
 *     ntA, ntW          128-row tiles of the stacked A rows of one adapter; of W
 *     n_used            adapters the plan is for
 *     GA, GW            A blocks (the shrink), W blocks (stream-K over the W units)
 *     smaxW             partial-sum slots per W tile (the most blocks sharing one tile)
 *     off_cnt, off_pa, pa_bytes, off_pw, pw_bytes, off_th, t_bytes, off_tl, total
 *                       workspace layout: counters, A partials, W partials, T_hi, T_lo,
 *                       total bytes
 *
 * Returns the number of values the plan has (18), or 0 when the shape is not on
 * the decode path or an argument is invalid.
 */
int32_t lora_decode_plan_describe(int64_t M, int64_t N, int64_t K, int32_t rank, int32_t n_slices,
                                  const int64_t* slice_n, int32_t n_used, int64_t* out, int32_t n_out);

#ifdef __cplusplus
}
#endif

#endif /* LORA_PROJ_H */
