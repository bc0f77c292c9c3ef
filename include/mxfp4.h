/*
 * mxfp4.h -- C ABI of the MI355X (gfx950) MXFP4 GEMM library (libmxfp4.so).
 *
 *   C[M,N] (bf16) = Q(A[M,K] bf16) * B[N,K]^T
 *
 * A is quantized at call time to MXFP4: one e8m0 power-of-two scale per 32
 * consecutive K elements, e2m1 elements; B is MXFP4 prepared once, offline,
 * in the preshuffled layouts below.
 *
 * Sources (web pages, each a diff between two versions of a submission to
 * the "amd-mxfp4-mm" leaderboard; cited by submission number):
 *   submission 608632  (hardware FP4 convert; kernel v7; bypass launchers)
 *   submission 610679  (constexpr kernels; split-K launcher + reduce)
 *   submission 711914  (three-path dispatch; standalone quant kernel)
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers (hipMalloc'ed or equivalent) unless said
 *     otherwise.  The caller owns every buffer; the library never frees or
 *     retains them beyond the call.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *     Work is enqueued asynchronously; no entry point synchronizes the host.
 *   - Arguments are checked on the host before anything is enqueued; a
 *     failed check returns an error and enqueues nothing.  Device faults
 *     surface at the caller's next synchronization, as usual in HIP.
 *   - Pointers that the kernels read or write in 16-byte vectors (bf16 and
 *     packed FP4 matrices, and C) must be 16-byte aligned.
 *   - Inputs must be finite; NaN/Inf in A or B are outside the method.
 */
#ifndef MXFP4_H
#define MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define MXFP4_API __attribute__((visibility("default")))
#else
#define MXFP4_API
#endif

typedef void *mxfp4_stream_t; /* a hipStream_t */

typedef enum {
    MXFP4_OK = 0,
    MXFP4_ERR_INVALID_ARG = 1, /* null pointer, size <= 0, misaligned pointer  */
    MXFP4_ERR_UNSUPPORTED = 2, /* shape outside what the kernels handle         */
    MXFP4_ERR_WORKSPACE = 3,   /* caller workspace too small                    */
    MXFP4_ERR_HIP = 4          /* a HIP call or kernel launch failed            */
} mxfp4_status_t;

/* ------------------------------------------------------------------------ */
/* Sizes (host only, pure).                                                  */
/* ------------------------------------------------------------------------ */

/* Packed e2m1 bytes of a [rows, K] matrix: rows * K / 2.  Element 2i of a
 * row sits in the low nibble of byte i, element 2i+1 in the high nibble
 * (submission 608632, _hw_mxfp4_quant_op, step 3). */
MXFP4_API size_t mxfp4_packed_bytes(int64_t rows, int64_t K);

/* Natural-layout scales: rows * (K / 32) bytes, row-major. */
MXFP4_API size_t mxfp4_raw_scale_bytes(int64_t rows, int64_t K);

/* Shuffled scales: pad256(rows) * pad8(K / 32) bytes, viewed as
 * [pad256(rows) / 32, pad8(K / 32) * 32] (submission 608632, bypass
 * launchers, the s0/s1 padding of the scale buffer).  Byte of (row, g):
 *   row = 32*r0 + 16*r1 + r2,  g = 8*k0 + 4*k1 + k2,
 *   r1 + 2*k1 + 4*r2 + 64*k2 + 256*k0 + r0 * 32 * pad8(K/32)
 * (submission 608632, _shuffle_scales; submission 711914, the address
 * arithmetic of _standalone_quant_kernel).  Padding bytes are 127 (2^0),
 * the fill submission 711914 gives its scale buffer. */
MXFP4_API size_t mxfp4_shuffled_scale_bytes(int64_t rows, int64_t K);

/* Workspace bytes mxfp4_gemm_ex needs for this shape (split-K partial sums,
 * per-tile tickets and, for the large-M kernel, the quantized A operand); 0
 * when the chosen schedule needs none.  (Not on the pages: their split-K
 * launcher allocates its partial-sum buffer per call; a C library exposes
 * the size so the caller can own the memory.) */
MXFP4_API size_t mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* ------------------------------------------------------------------------ */
/* Quantize a bf16 matrix to MXFP4.                                           */
/* Per 32-element group along K: amax = max |x| in f32; R = (bits(amax) +    */
/* 0x200000) & 0xFF800000; scale byte s = clamp(exponent(R) - 2, 0, 254)     */
/* (submission 608632, _hw_mxfp4_quant_op, steps 1-2).  Each element is      */
/* x / 2^(s-127) rounded to the nearest e2m1 value, ties to even, saturated  */
/* at 6, sign kept (submission 711914, _mxfp4_quant_tile).                   */
/*                                                                           */
/*   x_bf16   [rows, K] bf16, row-major, 16-byte aligned          (input)    */
/*   q        [rows, K/2] bytes, 16-byte aligned                  (output)   */
/*   scales   raw [rows, K/32] (shuffled_scales == 0), or the shuffled,      */
/*            padded buffer of mxfp4_shuffled_scale_bytes bytes, padding      */
/*            written as 127 (shuffled_scales != 0)                (output)   */
/* Errors: INVALID_ARG (null, rows < 1, K < 32, misaligned x or q);          */
/*         UNSUPPORTED (K % 32 != 0, sizes beyond 2^31 bytes).               */
/* ------------------------------------------------------------------------ */
MXFP4_API mxfp4_status_t mxfp4_quantize(const void *x_bf16, int64_t rows, int64_t K, void *q, void *scales,
                              int shuffled_scales, mxfp4_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Rearrange quantized B into the layouts mxfp4_gemm reads.                  */
/*   bq          [N, K/2] packed e2m1, natural layout, 16-byte aligned        */
/*   bs_raw      [N, K/32] raw scales                                         */
/*   bq_shuffled [N/16, (K/2)*16] bytes: 16-row x 16-byte tiles, each 256    */
/*               contiguous bytes row-major, tiles of a 16-row group          */
/*               consecutive along K, groups consecutive:                     */
/*               out[g*(K/2)*16 + t*256 + n*16 + j] = bq[16g+n][16t+j]        */
/*               (the layout whose inverse submissions 608632, kernel v7,     */
/*               and 711914, _unshuffle_b_preshuffle, print)                  */
/*   bs_shuffled mxfp4_shuffled_scale_bytes(N, K) bytes, as above             */
/* Errors: INVALID_ARG (null, N < 1, K < 32, misaligned);                    */
/*         UNSUPPORTED (N % 16 != 0, K % 32 != 0, sizes beyond 2^31 bytes). */
/* ------------------------------------------------------------------------ */
MXFP4_API mxfp4_status_t mxfp4_preshuffle_b(const void *bq, const void *bs_raw, int64_t N, int64_t K, void *bq_shuffled,
                                  void *bs_shuffled, mxfp4_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Prepare B for mxfp4_gemm in one launch: quantize bf16 B (as               */
/* mxfp4_quantize) and write the codes and scales straight into the layouts */
/* mxfp4_preshuffle_b produces.  The result is byte-identical to            */
/* mxfp4_quantize followed by mxfp4_preshuffle_b.  (Submission 608632's      */
/* patched input generator prepares B offline: quantize, then shuffle the    */
/* codes and the scales.)                                                    */
/*   b_bf16      [N, K] bf16, row-major, 16-byte aligned          (input)    */
/*   bq_shuffled [N/16, (K/2)*16] bytes, as mxfp4_preshuffle_b     (output)   */
/*   bs_shuffled mxfp4_shuffled_scale_bytes(N, K) bytes, padding 127 (output) */
/* Errors: INVALID_ARG (null, N < 1, K < 32, misaligned);                    */
/*         UNSUPPORTED (N % 16 != 0, K % 32 != 0, sizes beyond 2^31 bytes). */
/* ------------------------------------------------------------------------ */
MXFP4_API mxfp4_status_t mxfp4_prepare_b(const void *b_bf16, int64_t N, int64_t K, void *bq_shuffled,
                                         void *bs_shuffled, mxfp4_stream_t stream);

/* ------------------------------------------------------------------------ */
/* The GEMM with A already quantized: C = dequant(Aq, As) * B^T, bf16 out.   */
/* A quantized once can serve several GEMMs.  (Submission 711914 quantizes   */
/* A with a standalone kernel and hands FP4 A and its shuffled scales to the */
/* GEMM for large M; mxfp4_quantize with shuffled_scales = 1 writes exactly  */
/* these inputs.)  Same C as mxfp4_gemm on the bf16 A when both run the same */
/* pre-quantized schedule; only such schedules run here.  Below 256 rows     */
/* the GEMM reads Aq and As as they are, in one launch; the large-M kernel   */
/* first repacks them into its own operand layout in the workspace.          */
/*   Aq      [M, K/2] packed e2m1, natural layout, 16-byte aligned (input)   */
/*   As      shuffled scales, mxfp4_shuffled_scale_bytes(M, K) bytes (input) */
/*   Bq_sh, Bs_sh, C, M, N, K, stream: as mxfp4_gemm                         */
/* Uses the library-owned workspace of (device, stream), like mxfp4_gemm.    */
/* Errors: as mxfp4_gemm; INVALID_ARG also for a null As.                    */
/* ------------------------------------------------------------------------ */
MXFP4_API mxfp4_status_t mxfp4_gemm_q(const void *Aq, const void *As, const void *Bq_sh, const void *Bs_sh, void *C,
                                      int64_t M, int64_t N, int64_t K, mxfp4_stream_t stream);

/* Name of the schedule mxfp4_gemm_q would run for a shape (a pre-quantized  */
/* one), or NULL if none covers it.  Thread-local static string.            */
MXFP4_API const char *mxfp4_gemm_q_schedule_name(int64_t M, int64_t N, int64_t K);

/* ------------------------------------------------------------------------ */
/* The fused GEMM: quantize A on the fly (as mxfp4_quantize), multiply by    */
/* the preshuffled B with scaled FP4 matrix instructions, accumulate in f32, */
/* round to bf16 (nearest even) and store C.  (submission 608632, kernel v7: */
/* quant of the bf16 A tile inside the K loop, scaled e2m1 x e2m1 dot into   */
/* an f32 accumulator, bf16 store; submission 610679, split-K kernel +       */
/* reduce: here the reduction happens inside the same launch.)               */
/*                                                                           */
/*   A       [M, K] bf16 row-major, 16-byte aligned                (input)   */
/*   Bq_sh   bq_shuffled of mxfp4_preshuffle_b, 16-byte aligned    (input)   */
/*   Bs_sh   bs_shuffled of mxfp4_preshuffle_b, 16-byte aligned    (input)   */
/*   C       [M, N] bf16 row-major, fully overwritten; must not alias the    */
/*           inputs; 16-byte aligned                                (output) */
/* mxfp4_gemm uses a library-owned workspace per (device, stream), created   */
/* on the first call for a shape that needs more (that call allocates and    */
/* zeroes it with a fill kernel on `stream`, never a memset; later calls do  */
/* not allocate).  A workspace that a larger one replaces is not freed: it   */
/* stays allocated until the process ends, so a HIP graph captured before    */
/* the growth still replays into valid memory (growth at least doubles the   */
/* size, so what stays behind is at most about the live buffer's size).      */
/* The device is the calling thread's current device, which `stream` must    */
/* belong to.  Results are deterministic: the split-K partial sums */
/* are added in a fixed order (unless an "_at" schedule is forced by         */
/* mxfp4_set_schedule_override: its float atomics add in arrival order).     */
/* Errors: INVALID_ARG (null, M/N/K < 1, misaligned);                        */
/*         UNSUPPORTED (K % 64 != 0 -- the harness's precondition, submission */
/*         608632 input generator --, N % 32 != 0, sizes beyond 2^31 bytes); */
/*         HIP (allocation or launch failure).                               */
/* ------------------------------------------------------------------------ */
MXFP4_API mxfp4_status_t mxfp4_gemm(const void *A, const void *Bq_sh, const void *Bs_sh, void *C, int64_t M, int64_t N,
                          int64_t K, mxfp4_stream_t stream);

/* As mxfp4_gemm with a caller-owned workspace of at least
 * mxfp4_gemm_workspace_bytes(M, N, K) bytes, 256-byte aligned.  (Not on the
 * pages: the caller-owned form of the workspace mxfp4_gemm keeps itself, for
 * callers that manage memory, such as graph capture on several streams.)  Its first
 * 65536 bytes hold one ticket word per output tile and must be zero before
 * the first use (zero-fill the whole buffer once); every call leaves them at
 * zero again, so later calls -- also for other shapes -- need no clearing.
 * The rest holds f32 partial sums.  Calls that share a workspace must not
 * overlap in time.
 * Errors: as mxfp4_gemm, plus WORKSPACE (too small or null when needed). */
MXFP4_API mxfp4_status_t mxfp4_gemm_ex(const void *A, const void *Bq_sh, const void *Bs_sh, void *C, int64_t M, int64_t N,
                             int64_t K, void *workspace, size_t workspace_bytes, mxfp4_stream_t stream);

/* ------------------------------------------------------------------------ */
/* mxfp4_gemm without any allocation, for callers that cannot allocate:     */
/* code under HIP graph capture, tight serving loops, harnesses that forbid */
/* hipMalloc.  Same arguments, results and errors as mxfp4_gemm.  Instead of */
/* a workspace it uses a scratch array of MXFP4_NOALLOC_SCRATCH_BYTES that  */
/* the library holds in device memory, one per GPU, from the first call on  */
/* that GPU until the process ends.  It calls no hipMalloc, hipFree or       */
/* other allocating routine; the first call on a GPU looks the array up and  */
/* clears its ticket words with a fill kernel on `stream`.                   */
/* Every call on a GPU shares that GPU's array, which keeps the last call's  */
/* contents: calls that overlap in time on one GPU (concurrent streams,      */
/* threads) race and must be serialized by the caller.                       */
/* Errors: as mxfp4_gemm, plus WORKSPACE when the schedule chosen for the    */
/* shape needs more than MXFP4_NOALLOC_SCRATCH_BYTES (large M times long K:  */
/* the quantized A operand of the large-M kernel, about M * K * 17/32 bytes, */
/* or split-K partial sums).                                                 */
/* ------------------------------------------------------------------------ */
#define MXFP4_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)
MXFP4_API mxfp4_status_t mxfp4_gemm_noalloc(const void *A, const void *Bq_sh, const void *Bs_sh, void *C, int64_t M,
                                            int64_t N, int64_t K, mxfp4_stream_t stream);

/* Create the library-owned workspace for (M, N, K) on `stream` ahead of time
 * (so that no later mxfp4_gemm call allocates, e.g. under graph capture).
 * (Not on the pages: their launchers pre-warm compiled variants; this is the
 * same idea for the workspace.) */
MXFP4_API mxfp4_status_t mxfp4_reserve(int64_t M, int64_t N, int64_t K, mxfp4_stream_t stream);

/* Human-readable name of a status code (static storage).  (Not on the
 * pages, whose errors are Python exceptions; the C form of their messages.) */
MXFP4_API const char *mxfp4_status_string(mxfp4_status_t status);

/* Name of the last HIP error (hipGetErrorName) that an MXFP4_ERR_HIP result */
/* of this thread came from, or "hipSuccess"; a static string.               */
MXFP4_API const char *mxfp4_last_hip_error(void);

/* Name of the kernel schedule mxfp4_gemm picks for a shape (thread-local
 * storage, valid until the next call on the thread), e.g.
 * "mt1_nt1_wn2_wk4_kpw1_split2" (16-row M tiles, 16-column subtiles per
 * wave, waves along N, waves along K, K steps per wave, workgroups per
 * output tile along K); NULL if the shape is unsupported.  The choice: the
 * measured best for the shapes of a built-in table, else the least
 * estimated time among the compiled fused kernels (and, above 64 rows or
 * for K too long for them, the large-M kernels), the estimate growing with
 * the 128-byte lines each CU must request. */
MXFP4_API const char *mxfp4_gemm_schedule_name(int64_t M, int64_t N, int64_t K);

/* Process-wide choice of the e2m1 encoder used by mxfp4_quantize and the
 * fused GEMM: 0 = the hardware convert (default), 1 = a software encoder
 * (the pages keep such a fallback next to the hardware path: submission
 * 608632, the warmup self-check and USE_HW_QUANT switch).  Both produce
 * identical bytes.  Not to be changed while calls are in flight.
 * Errors: INVALID_ARG for any other mode. */
MXFP4_API mxfp4_status_t mxfp4_set_quant_mode(int mode);

/* Process-wide schedule override for mxfp4_gemm, by the name format of
 * mxfp4_gemm_schedule_name (for tuning sweeps); NULL or "" restores the
 * built-in choice.  Besides the names the built-in choice gives, it takes
 * the split-K epilogues the built-in choice never picks:
 *   "..._split<n>_at" (or "_r8_at"): the partial tiles are added with f32
 *       atomics into a workspace tile that a separate launch zero-fills
 *       first (submission 711914, the fused large-K kernel, adds into a
 *       zeroed f32 C); the last workgroup of a tile casts it to bf16.  Not
 *       deterministic: the additions happen in arrival order.
 *   "mt.._kpw<k>_streamk<G>" (or "_r8"): stream-K, G workgroups each taking
 *       an equal run of the tiles x K steps iterations; deterministic.
 *   "widel_...": the large-M kernel with B staged through LDS.
 * A call whose shape the override cannot serve returns UNSUPPORTED.
 * Errors: INVALID_ARG for a name no compiled kernel matches. */
MXFP4_API mxfp4_status_t mxfp4_set_schedule_override(const char *name);

/* Tuning: the names of every compiled schedule that can serve (M, N, K),
 * one per line, for timing with mxfp4_set_schedule_override.  Listed: the
 * fused kernels with the ticketed split epilogue at each split 1..16 that
 * covers K (for quantized_a != 0, the ones that read A as codes, as
 * mxfp4_gemm_q does), then the large-M kernels at splits 1..8; no split
 * larger than K's count of 128-wide steps.  The
 * built-in choice is always among them.  Host-only; no GPU needed.
 * Writes at most `cap` bytes into `buf`, always NUL-terminated when
 * cap > 0 (names are cut only at the cap), and returns the length the whole
 * list needs, without the NUL: call once with cap = 0 to size the buffer.
 * Returns 0 for a shape outside the ABI (see mxfp4_gemm's errors). */
MXFP4_API size_t mxfp4_list_schedules(int64_t M, int64_t N, int64_t K, int quantized_a, char *buf, size_t cap);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
