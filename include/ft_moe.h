/*
 * ft_moe.h -- C ABI of the routed MoE FFN layer with a resident-expert cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer, one call per step:
 *   ft_moe_route        router logits (optional) + top-k + gating weights
 *   ft_moe_permute      token-to-expert permutation into per-expert segments
 *   ft_moe_grouped_ffn  SwiGLU expert FFN over the segments, weights read
 *                       through a resident-expert slot table
 *   ft_moe_combine      weighted combine of the expert rows back to tokens
 *   ft_expert_cache_*   the shared (layer, expert) LRU slot table on the
 *                       device, with misses filled from pinned host memory
 *
 * Source of the method: the FreeToken pages.  A router activates a small
 * subset of the experts for each token (6 of 256 routed experts per layer in
 * their example); the full expert set lives in host memory and GPU memory is
 * an elastic cache of whole (layer, expert) entries under one LRU policy
 * shared by every MoE layer; hits run on the GPU from the cached copy and
 * misses are moved over PCIe from pinned host memory (FreeToken linux page,
 * "Cómo gestiona FreeToken la memoria MoE"; FreeToken quantization page,
 * "Cómo se desplazan los pesos MoE cuantizados por la memoria"; FreeToken
 * rtx 4090 page, "Cómo funciona la jerarquía de memoria MoE").  The pages do
 * not write the layer arithmetic; the textbook reading used here is stated at
 * each call.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless marked "host".  The caller owns every
 *    buffer; a call borrows its buffers until the work it enqueued finishes.
 *  - Arguments are validated synchronously before anything is enqueued.  On an
 *    error nothing is enqueued and no state changes.  Work is enqueued on
 *    `stream` and the call returns without waiting, except
 *    ft_expert_cache_step, which waits once for its miss list (see there).
 *  - Return value: FT_OK (0) or a negative ft_status.  ft_last_error() gives a
 *    text for the last failing call on the calling host thread.  Faults of
 *    enqueued work surface at the caller's next synchronisation.
 *  - Hot-path calls (route, permute, grouped FFN, combine, the cache's step,
 *    plan / fill, prefetch and CPU-miss calls) never allocate device or host
 *    memory.  Scratch memory is passed in as `workspace`, sized by
 *    ft_workspace_bytes(); the cache allocates its state at create, its
 *    event ring at ft_expert_cache_set_trace and its CPU-miss buffers at
 *    ft_expert_cache_set_split.
 *  - Row-major layouts throughout; [a, b] means a rows of b contiguous elements.
 */
#ifndef FT_MOE_H
#define FT_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ft_status;
enum {
  FT_OK = 0,
  FT_EINVAL = -1,     /* null pointer, bad shape, bad enum, misaligned buffer */
  FT_ENOTSUP = -2,    /* valid request outside what the kernels implement     */
  FT_ECAPACITY = -3,  /* a cache step needs more distinct experts than slots  */
  FT_EHIP = -4        /* a HIP runtime call failed                            */
};

/* Text of the last error on this host thread ("" if none).  Owned by the library. */
const char *ft_last_error(void);

/* Library version string, e.g. "ftmoe 0.1 gfx950". */
const char *ft_version(void);

typedef enum { FT_F32 = 0, FT_BF16 = 1, FT_MXFP4 = 2, FT_NVFP4 = 3 } ft_dtype;
typedef enum { FT_SOFTMAX = 0, FT_SIGMOID = 1 } ft_gating;

/* slot_of_expert value for an expert whose rows a grouped-FFN call must leave
 * untouched (another call computes them; see ft_expert_cache_step_split).
 * Any other negative slot means "not resident": its rows are written as NaN. */
#define FT_SLOT_SKIP (-2)

/* ------------------------------------------------------------------------ */
/* Expert blob layout                                                        */
/* ------------------------------------------------------------------------ */
/*
 * One cache entry is one whole (layer, expert) pair, stored as one contiguous
 * blob with the same layout in host memory and in a GPU slot (FreeToken rtx
 * 4090 page, "Cómo funciona la jerarquía de memoria MoE": an entry is a whole
 * expert under one logical mapping on CPU and GPU).
 *
 * Blob = [gate][up][down] (+ for MXFP4: [gate scales][up scales][down scales]),
 * each part starting at a 256-byte boundary, expert_bytes rounded up to 4 KiB.
 *   gate, up : [I, H]   (contraction axis H contiguous)
 *   down     : [H, I]   (contraction axis I contiguous)
 * FT_F32 / FT_BF16: elements of that type.
 * FT_MXFP4 (OCP Microscaling v1.0): codes [rows, K/2] bytes, element 2i in
 *   bits 3:0 and element 2i+1 in bits 7:4 of byte i, FP4 E2M1 values;
 *   scales [rows, K/32] bytes, E8M0 (2^(byte-127)), one per 32 consecutive
 *   elements of a row along its contraction axis K.
 * FT_NVFP4 (named on FreeToken's quantization page, results and hardware
 *   tables; format as NVIDIA publishes it): the same codes; scales
 *   [rows, K/16] bytes, FP8 E4M3 (OCP), one per 16 consecutive elements; and
 *   three fp32 tensor scales (gate, up, down) at off_tscale.  Element =
 *   E2M1 x E4M3(block scale) x tensor scale.
 */
typedef struct {
  int32_t wdtype;        /* ft_dtype of the expert weights                     */
  int32_t H, I;          /* hidden size, expert intermediate size              */
  int32_t reserved;
  uint64_t expert_bytes; /* bytes of one blob (a multiple of 4096)             */
  uint64_t off_gate, off_up, off_down;      /* byte offsets of the three parts */
  uint64_t off_sgate, off_sup, off_sdown;   /* MXFP4 / NVFP4 scale parts (0 otherwise) */
  uint64_t off_tscale;   /* NVFP4: 3 fp32 tensor scales (gate, up, down); 0 otherwise */
} ft_expert_layout;

/* Fill *out for experts of type wdtype.  Host only, pure.
 * Errors: FT_EINVAL (out NULL, H or I < 1, unknown dtype, MXFP4 with H or I
 * not a multiple of 32, NVFP4 with H or I not a multiple of 16). */
ft_status ft_expert_layout_init(int32_t wdtype, int32_t H, int32_t I, ft_expert_layout *out);

/* ------------------------------------------------------------------------ */
/* Routing                                                                    */
/* ------------------------------------------------------------------------ */
/*
 * ft_moe_route -- a router picks k of the E routed experts per token (FreeToken
 * linux page, "Cómo gestiona FreeToken la memoria MoE").
 *
 * If w_router != NULL: logits[t, e] = sum_h x[t, h] * w_router[e, h] is computed
 *   with fp32 accumulation and written to `logits` [T, E] fp32.
 *   x [T, H] and w_router [E, H] are both of type x_dtype (FT_F32 or FT_BF16).
 * If w_router == NULL: `logits` [T, E] fp32 is read (x and H are ignored).
 * topk_ids [T, k] int32: per token the k largest logits in descending order,
 *   the lower expert index first on equal logits (-0.0 equals +0.0).
 * topk_w [T, k] fp32: FT_SOFTMAX -> softmax over all E of the token's logits,
 *   taken at the picked experts; FT_SIGMOID -> sigmoid of the picked logits.
 *   renormalize != 0 divides the k weights by their sum.
 * Limits: 1 <= k <= E <= 1024 (else FT_ENOTSUP).  T = 0 is a no-op.
 * Buffers 16-byte aligned; with w_router and FT_BF16, H must be a multiple
 * of 128 (FT_ENOTSUP otherwise).
 * NaN or infinite logits are outside the contract.
 */
ft_status ft_moe_route(const void *x, int32_t x_dtype, const void *w_router, float *logits,
                       int32_t T, int32_t H, int32_t E, int32_t k, int32_t gating,
                       int32_t renormalize, int32_t *topk_ids, float *topk_w,
                       hipStream_t stream);

/*
 * ft_moe_permute -- group the routed rows by expert.  Flat row r = t*k + j is
 * token t's j-th pick.  expert_offsets [E+1]: exclusive prefix sum of the
 * per-expert row counts (expert_offsets[E] = T*k).  sorted_rows [T*k]: the rows
 * of expert 0, then expert 1, ..., ascending within each segment.  row_pos
 * [T*k]: the inverse, row_pos[sorted_rows[i]] = i.
 * topk_ids must hold values in 0..E-1 (out-of-range ids are a caller error: the
 * kernel ignores such rows and the outputs are then unspecified).
 * workspace: ft_workspace_bytes(FT_WS_PERMUTE, T, k, E, 0, 0) bytes (may be 0
 * for small T*k, then workspace may be NULL).
 * Limits: 1 <= E <= 4096, T*k < 2^31.
 */
ft_status ft_moe_permute(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                         int32_t *expert_offsets, int32_t *sorted_rows, int32_t *row_pos,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ft_moe_route_permute -- ft_moe_route followed by ft_moe_permute on the same
 * stream, with the same arguments, results and errors.  When 1 <= T <= 16 and
 * T*k <= 2048 (small decode batches, where per-launch latency is most of the
 * cost of routing) top-k, gating and the permutation run as one launch after
 * the router logits; otherwise it makes the two calls.
 * workspace: ft_workspace_bytes(FT_WS_ROUTE_PERMUTE, T, k, E, 0, 0) bytes
 * (ft_moe_permute's; may be 0, then workspace may be NULL).
 */
ft_status ft_moe_route_permute(const void *x, int32_t x_dtype, const void *w_router, float *logits,
                               int32_t T, int32_t H, int32_t E, int32_t k, int32_t gating,
                               int32_t renormalize, int32_t *topk_ids, float *topk_w,
                               int32_t *expert_offsets, int32_t *sorted_rows, int32_t *row_pos,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Expert FFN                                                                 */
/* ------------------------------------------------------------------------ */
/*
 * ft_moe_grouped_ffn -- every routed row runs its expert from the expert's
 * resident copy (FreeToken quantization page, "Cómo se desplazan los pesos MoE
 * cuantizados por la memoria": hits run on the GPU from the cache).  The
 * expert is a SwiGLU FFN (Shazeer 2020, no biases):
 *     y = (silu(x Wg^T) * (x Wu^T)) Wd^T,   silu(z) = z / (1 + e^-z).
 *
 * Segment e = rows expert_offsets[e] .. expert_offsets[e+1]-1 of the permuted
 * order; its row i is token sorted_rows[i] / k.  Expert e's blob starts at
 *   slot_pool + slot_of_expert[e] * L->expert_bytes
 * (slot_of_expert == NULL means slot e).  slot_pool holds n_slots blobs
 * (n_slots >= 1; >= E when slot_of_expert is NULL).  A segment whose slot is
 * FT_SLOT_SKIP is left untouched (its hidden and y rows are not written); a
 * non-empty segment with another negative slot, or a slot >= n_slots, is a
 * caller error: nothing is read for it and its y rows are written as NaN.
 * x [T, H] of x_dtype (FT_F32 with FT_F32 weights, FT_BF16 with FT_BF16 or
 *   FT_MXFP4 weights).
 * y_rows [T*k, H] fp32, permuted order (row i belongs to sorted_rows[i]).
 * shared_blob (nullable): one more expert in the same layout, applied to every
 *   token with weight 1, written to y_shared [T, H] fp32 (required iff
 *   shared_blob != NULL).
 * mode, low byte:
 *   FT_FFN_EXACT (0) -- MXFP4 weights decoded exactly to bf16, bf16 MFMA,
 *     fp32 accumulation; the SwiGLU hidden vector is rounded to bf16 before
 *     the down projection.
 *   FT_FFN_NATIVE_MX (1, FT_MXFP4 weights only; otherwise FT_ENOTSUP) -- the
 *     matrix unit takes the MXFP4 weights as stored: x and the bf16-rounded
 *     hidden vector are quantized to MXFP8 E4M3 exactly as ft_mxfp8_quantize
 *     does, and both products run as block-scaled FP8 x FP4 MFMA with fp32
 *     accumulation.  The results differ from FT_FFN_EXACT by the activation
 *     quantization (a few percent); they match a float64 evaluation of the
 *     same quantized operands.
 *   Other values: FT_ENOTSUP.
 * mode, stage bits: FT_FFN_GATE_UP_ONLY runs only the gate/up + SwiGLU stage
 *   (y is not written); FT_FFN_DOWN_ONLY runs only the down projection from
 *   the hidden rows in `workspace` (left there by a FT_FFN_GATE_UP_ONLY call
 *   with the same arguments, or written by the caller).  Neither bit: both
 *   stages.  Both bits: FT_EINVAL.  For bf16 and MXFP4 weights the hidden
 *   rows are bf16 [T*k (+T), I] at the start of the workspace: row p of the
 *   permuted order, then the shared expert's row of token t at T*k + t; fp32
 *   weights keep fp32 rows there.
 * workspace: ft_workspace_bytes(FT_WS_FFN, T, k, E, H, I) bytes.
 * Limits: FT_BF16 weights need H, I multiples of 128; FT_MXFP4 multiples of
 *   256; E <= 4096.  MXFP4 scale bytes must lie in 2..252 (every decoded value
 *   is then an exact bf16).  Buffers 16-byte aligned, slot_pool and blobs
 *   256-byte aligned.
 */
enum { FT_FFN_EXACT = 0, FT_FFN_NATIVE_MX = 1 };
enum { FT_FFN_GATE_UP_ONLY = 0x100, FT_FFN_DOWN_ONLY = 0x200 };
ft_status ft_moe_grouped_ffn(const ft_expert_layout *L, const void *slot_pool, int32_t n_slots,
                             const int32_t *slot_of_expert, const void *shared_blob,
                             const void *x, int32_t x_dtype, int32_t T, int32_t k, int32_t E,
                             const int32_t *expert_offsets, const int32_t *sorted_rows,
                             float *y_rows, float *y_shared, int32_t mode,
                             void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * ft_moe_grouped_ffn_noalloc -- ft_moe_grouped_ffn with the same arguments,
 * results and errors, minus the workspace: for callers that cannot allocate
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The workspace is a static device array of
 * ft_noalloc_scratch_bytes() bytes (16 MiB) that each GPU the library runs on
 * holds until the process ends; its address on a GPU is resolved on the first
 * call there.  The call allocates nothing.
 * A call whose ft_workspace_bytes(FT_WS_FFN, T, k, E, H, I) exceeds that size
 * returns FT_ECAPACITY and enqueues nothing (decode batches fit: e.g. 64
 * tokens of H=2048, I=768, top-8, or 32 tokens of H=4096, I=2048, top-6 with a
 * shared expert, in either mode).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other host threads)
 * race and must be ordered by the caller.  FT_FFN_DOWN_ONLY reads the hidden
 * rows that the last FT_FFN_GATE_UP_ONLY call of this entry point on the GPU
 * left there.
 */
ft_status ft_moe_grouped_ffn_noalloc(const ft_expert_layout *L, const void *slot_pool, int32_t n_slots,
                                     const int32_t *slot_of_expert, const void *shared_blob,
                                     const void *x, int32_t x_dtype, int32_t T, int32_t k, int32_t E,
                                     const int32_t *expert_offsets, const int32_t *sorted_rows,
                                     float *y_rows, float *y_shared, int32_t mode, hipStream_t stream);

/* Bytes of the static scratch array of ft_moe_grouped_ffn_noalloc (per GPU). */
size_t ft_noalloc_scratch_bytes(void);

/*
 * ft_read_checksum -- *sink ^= the XOR of the 32-bit words of buf[0 .. bytes),
 * on the device, the buffer read once in whole 128-byte lines.  It is the
 * plain read that bounds a weight stream (the pages' decode reads every
 * activated expert's weights once per token: FreeToken 290b model page, "Cómo
 * gestiona FreeToken el prellenado y la decodificación"), timed beside the
 * decode kernels, and a check that a copied expert blob arrived whole.
 * buf: device memory, 16-byte aligned; bytes a multiple of 16, at most 2^31
 * (larger buffers: checksum slices and XOR the results); sink: 4 device
 * bytes, not cleared (start it at 0).  The result does not depend on the
 * launch shape.  Errors before anything is enqueued: FT_EINVAL (NULL or
 * misaligned pointer, bytes not a multiple of 16), FT_ENOTSUP (above 2 GiB).
 */
ft_status ft_read_checksum(const void *buf, uint64_t bytes, uint32_t *sink, hipStream_t stream);

/*
 * Instruction paths of the host expert kernel (ft_cpu_expert_ffn,
 * ft_cpu_miss_rows).  Both compute the same products; they differ only in the
 * order of fp32 additions.
 */
enum {
  FT_CPU_ISA_QUERY = -1,  /* ft_cpu_isa: report only */
  FT_CPU_ISA_BEST = 0,    /* the best the host supports (the default) */
  FT_CPU_AVX2 = 1,        /* AVX2 + FMA: activations widened to fp32 */
  FT_CPU_AVX512_BF16 = 2  /* AVX-512 BF16: bf16 pair dot products into fp32 */
};

/* Select (or query, FT_CPU_ISA_QUERY) the host kernel's path for the process;
 * *active (may be NULL) receives the path in use.  A path the host lacks ->
 * FT_ENOTSUP, nothing changed; an unknown request -> FT_EINVAL. */
ft_status ft_cpu_isa(int32_t request, int32_t *active);

/*
 * ft_cpu_expert_ffn -- one expert's SwiGLU FFN on the host CPU, for misses the
 * hybrid split leaves to the CPU (FreeToken 290b model page, "Ejecución
 * híbrida": a miss may run directly on the CPU; the CPU expert kernel's
 * effective host bandwidth is the B_h of the split).  Same arithmetic as the
 * exact GPU mode: weights decoded exactly, fp32 accumulation, the hidden
 * vector rounded to bf16 before the down projection.
 * blob: HOST pointer to one expert blob in layout L (e.g. inside the pinned
 *   host bank), FT_BF16 or FT_MXFP4 weights with H and I multiples of 128
 *   (else FT_ENOTSUP).
 * x: HOST bf16 [n, H]; y: HOST fp32 [n, H] (written).  n >= 0.
 * n_threads: host threads (0: FTMOE_CPU_THREADS or all hardware threads); a
 *   persistent pool per thread count is kept for the process.
 * Synchronous: returns when y is written.  No GPU call is made.
 */
ft_status ft_cpu_expert_ffn(const ft_expert_layout *L, const void *blob, const void *x, int32_t n, float *y,
                            int32_t n_threads);

/*
 * ft_cpu_miss_rows -- the rows of a layer step's CPU misses (the experts
 * ft_expert_cache_cpu_misses lists) computed on the host, in the permuted
 * order of ft_moe_grouped_ffn's y_rows (same page and arithmetic as
 * ft_cpu_expert_ffn).  For each listed expert e, row i in
 * expert_offsets[e] .. expert_offsets[e+1]-1 is token sorted_rows[i] / k run
 * through expert (layer, e); y_rows[i] is written, no other row is touched.
 * All pointers are HOST pointers:
 *   bank: the host expert bank, blob (layer * E + e) at byte offset
 *     (layer * E + e) * L->expert_bytes (the layout ft_expert_cache_create takes);
 *   experts [n_experts], ids in [0, E); expert_offsets [E+1] with
 *     expert_offsets[0] = 0 and expert_offsets[E] = T*k, sorted_rows [T*k]
 *     (host copies of ft_moe_permute's outputs);
 *   x: bf16 [T, H]; y_rows: fp32 [T*k, H].
 * Errors: bad sizes, ids or offsets -> FT_EINVAL (nothing written); weights
 * other than bf16 / MXFP4 -> FT_ENOTSUP.  Synchronous; no GPU call is made.
 */
ft_status ft_cpu_miss_rows(const ft_expert_layout *L, const void *bank, int32_t layer, int32_t E,
                           const int32_t *experts, int32_t n_experts, const int32_t *expert_offsets,
                           const int32_t *sorted_rows, int32_t T, int32_t k, const void *x, float *y_rows,
                           int32_t n_threads);

/*
 * ft_mxfp8_quantize -- bf16 rows to MXFP8, the activation format of the native
 * MXFP4 mode (the pages name natively MXFP4-quantized routed experts, FreeToken
 * quantization page, "Formatos compatibles, hardware y perfil de rendimiento";
 * the format is OCP Microscaling Formats v1.0).  Each block of 32 consecutive
 * elements of a row gets the E8M0 scale byte b = floor(log2 amax) - 8 + 127
 * (amax = largest magnitude of the block; 0 for an all-zero block; clamped to
 * 0..254), and element v the FP8 E4M3 code nearest to v / 2^(b-127), ties to
 * the even code, magnitudes above 448 saturating to 448, the sign kept when v
 * rounds to zero.
 * x [n, K] bf16 with row pitch ldx elements (ldx >= K, a multiple of 8);
 * codes [n, K] bytes (row pitch K); scales [n, K / 32] bytes, scale j of a row
 * covering elements 32j .. 32j+31.  K a multiple of 32; x and codes 16-byte
 * aligned.  NaN or infinite inputs are outside the contract.
 */
ft_status ft_mxfp8_quantize(const void *x, int64_t ldx, int32_t n, int32_t K, uint8_t *codes,
                            uint8_t *scales, hipStream_t stream);

/*
 * ft_moe_combine -- out[t] = sum_{j<k} topk_w[t, j] * y_rows[row_pos[t*k + j]]
 * (+ y_shared[t] when y_shared != NULL), summed in j order and then the shared
 * row, in fp32; written as out_dtype (FT_F32, or FT_BF16 rounded to nearest
 * even).  y_rows [T*k, H] fp32, out [T, H].  H a multiple of 4; buffers
 * 16-byte aligned.
 * The pages say the router activates a few experts per token (FreeToken linux
 * page, "Cómo gestiona FreeToken la memoria MoE") but do not spell out how the
 * experts' outputs are joined; this call takes the usual reading: the
 * gating-weighted sum of the routed experts' rows (the scatter-add of the
 * permuted rows back to token order, in gather form), plus the shared
 * expert's row.
 */
ft_status ft_moe_combine(const float *y_rows, const float *topk_w, const int32_t *row_pos,
                         const float *y_shared, int32_t T, int32_t k, int32_t H,
                         int32_t out_dtype, void *out, hipStream_t stream);

/*
 * ft_moe_layer -- the whole routed MoE layer in one call: ft_moe_route_permute,
 * ft_moe_grouped_ffn and ft_moe_combine with the arguments below, the same
 * results (the routing outputs, out) and the same errors, all checked before
 * anything is enqueued.  The pages' decode produces tokens one at a time
 * (FreeToken 290b model page, "Cómo gestiona FreeToken el prellenado y la
 * decodificación"); with 1 <= T <= 4 tokens, exact mode, bf16 / MXFP4 / NVFP4
 * weights, E <= 256, k <= 16 and a contraction length the persistent decode
 * kernels cover, the layer runs as three launches instead of five:
 *   1. the router logits (when w_router != NULL);
 *   2. gate/up + SwiGLU, each workgroup taking top-k, gating and the
 *      permutation from the logits itself (one workgroup writes topk_ids,
 *      topk_w, expert_offsets, sorted_rows and row_pos);
 *   3. the down projection with the combine folded in: each output element
 *      is sum_j topk_w[t, j] * y_j (+ the shared expert's) in fp32, rounded
 *      once -- y_rows and y_shared are then NOT written.
 * With T = 1 and at most 8 down steps (k routed + the shared expert), steps 2
 * and 3 are one launch whose workgroups meet at a grid-wide wait.  Other
 * calls make the three calls in turn (y_rows / y_shared written as there);
 * with 17 or more tokens, at most 1024 routed rows and E <= 256, the routing
 * after the router is one launch: top-k over the grid, the permutation by the
 * workgroup that finishes last.  With 5 to 64 tokens, bf16 tokens and
 * E <= 256 the router's logits are computed in parts over H (partial sums
 * held at the start of the steps' workspace until the routing launch adds
 * them, in a fixed order, and writes logits).
 * An expert whose slot is negative (FT_SLOT_SKIP included) or >= n_slots
 * gives NaN outputs for the tokens that picked it.
 * Arguments: as for the three calls (x, x_dtype, w_router, logits, T, E, k,
 * gating, renormalize, topk_ids, topk_w, expert_offsets, sorted_rows, row_pos
 * as ft_moe_route_permute; L, slot_pool, n_slots, slot_of_expert,
 * shared_blob, y_rows, y_shared, mode as ft_moe_grouped_ffn -- mode without
 * stage bits; out_dtype, out as ft_moe_combine, H = L->H).
 * workspace: ft_workspace_bytes(FT_WS_LAYER, T, k, E, H, I) bytes, 256-byte
 * aligned.  Its first 8192 bytes are the wait area: the counters of the
 * one-token kernel's grid-wide wait and of the routing of 17 to 1024/k tokens
 * (top-k over the grid, the permutation by the workgroup that finishes
 * last).  Zero it once before the first call on a workspace; every
 * call leaves it ready for the next (the counters back at zero, the wait's
 * round words only counting up; a wait that gives up -- it never should --
 * writes NaN outputs and may leave the counters non-zero).  The rest is the
 * steps' workspace; after the call its start
 * (byte 8192) holds the bf16 hidden rows, as for ft_moe_grouped_ffn (for one
 * token on the one-token kernels: the picks' rows in pick order, then the
 * shared expert's).  Calls that share a workspace must not overlap.
 */
ft_status ft_moe_layer(const ft_expert_layout *L, const void *slot_pool, int32_t n_slots,
                       const int32_t *slot_of_expert, const void *shared_blob, const void *x, int32_t x_dtype,
                       const void *w_router, float *logits, int32_t T, int32_t E, int32_t k, int32_t gating,
                       int32_t renormalize, int32_t *topk_ids, float *topk_w, int32_t *expert_offsets,
                       int32_t *sorted_rows, int32_t *row_pos, float *y_rows, float *y_shared, int32_t mode,
                       int32_t out_dtype, void *out, void *workspace, size_t workspace_bytes,
                       hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Expert cache                                                               */
/* ------------------------------------------------------------------------ */
/*
 * One LRU over (layer, expert) entries, shared by all MoE layers, following the
 * router rather than fixed at start-up (FreeToken linux page, "Cómo gestiona
 * FreeToken la memoria MoE"; FreeToken rtx 4090 page, "Cómo funciona la
 * jerarquía de memoria MoE").  Hits run from the slot; misses are copied over
 * PCIe from the pinned host bank, the source of truth for every expert
 * (FreeToken quantization page, "Cómo se desplazan los pesos MoE cuantizados
 * por la memoria").  Miss rate = misses / routed expert reads (FreeToken 290b
 * model page, "Limitaciones, lista de comprobación y buenas prácticas").
 *
 * Update order inside one (layer, step) -- not on the pages, fixed here: the
 * needed set S = the distinct experts of the step's topk_ids, ascending.
 * Phase 1: every hit becomes most recently used (ascending expert id).
 * Phase 2: each miss (ascending) takes the least recently used slot holding
 * no member of S; empty slots count as oldest, lowest index first.
 */
typedef struct ft_expert_cache ft_expert_cache;  /* opaque */

typedef struct {
  uint64_t accesses;   /* distinct (layer, expert) reads, summed over steps */
  uint64_t hits, misses, evictions;
  uint64_t bytes_h2d;  /* bytes copied host -> device (miss and prefetch fills) */
  uint64_t steps;      /* successful ft_expert_cache_step calls             */
  uint64_t prefetch_fills;  /* entries brought in by ft_expert_cache_prefetch_layer */
  uint64_t cpu_misses;  /* misses left to the host CPU by the hybrid split (also in misses) */
  uint64_t cpu_ns;      /* host wall time inside ft_expert_cache_run_cpu_misses (waiting for the staged
                           inputs, the expert kernel, enqueueing the copy back): cpu_misses *
                           expert_bytes / cpu_ns is the effective B_h the decode loop sees */
  uint64_t trace_dropped;  /* events overwritten in the event ring (ft_expert_cache_set_trace) */
} ft_cache_stats;

/* One cache event, as recorded by the step (or layer prefetch) that produced it. */
typedef struct {
  int32_t step;        /* index of the ft_expert_cache_step call (from 0); a
                          prefetch records the number of steps before it    */
  int32_t layer;
  int32_t expert;
  int32_t hit;         /* 1 hit, 0 miss (filled), 4 miss left to the host CPU
                          (slot -1); prefetch: 3 already resident, 2 filled,
                          5 not prefetched for lack of room (slot -1)        */
  int32_t slot;
  int32_t evicted;     /* key layer*E + expert of the entry evicted, or -1    */
} ft_cache_event;

/*
 * Create a cache of `capacity` slots over n_layers x E experts of layout L.
 * slot_pool: device, capacity * L->expert_bytes bytes, 256-byte aligned,
 *   caller-owned, borrowed for the cache's lifetime.
 * host_bank: host, PINNED (hipHostMalloc), n_layers * E * L->expert_bytes
 *   bytes, blob of (layer l, expert e) at (l*E + e) * expert_bytes;
 *   caller-owned, borrowed for the cache's lifetime.
 * copy_stream: the stream the miss fills are enqueued on (not the NULL stream).
 * The cache allocates its small device state (about 16 B per key and slot)
 * and one pinned miss-list buffer here, and frees them in destroy.  It starts
 * empty.  Errors: FT_EINVAL (bad sizes, NULLs, host_bank not pinned host
 * memory, slot_pool not device memory), FT_EHIP.
 * Limits: capacity <= 65536, n_layers * E <= 2^20, E <= 4096.
 */
ft_status ft_expert_cache_create(const ft_expert_layout *L, int32_t n_layers, int32_t E,
                                 int32_t capacity, void *slot_pool, const void *host_bank,
                                 hipStream_t copy_stream, ft_expert_cache **out);

/*
 * Serve layer `layer` for the routing topk_ids [T, k] (device).
 * On return slot_of_expert [E] (device) holds, for every expert of the layer,
 * its slot or -1 if not resident; every expert in topk_ids is resident.
 * Synchronisation:
 *   1. the LRU kernel is enqueued on compute_stream; it writes the step's miss
 *      list into a pinned host buffer;
 *   2. the host waits for it (one host wait per call; it also drains earlier
 *      work of compute_stream, so no earlier kernel still reads a victim slot);
 *   3. one hipMemcpyAsync host->device per miss is enqueued on copy_stream;
 *   4. compute_stream is made to wait for those copies, and the call returns.
 * Kernels that read the slot pool must run on compute_stream (or be ordered
 * before the next ft_expert_cache_step call on it).
 * Errors: FT_EINVAL (bad layer, T, k, NULLs); FT_ECAPACITY if the step needs
 * more distinct experts than there are slots -- detected by the kernel; the
 * cache state is then unchanged; FT_EHIP.  topk_ids out of 0..E-1 -> FT_EINVAL
 * (detected by the kernel, state unchanged).
 */
ft_status ft_expert_cache_step(ft_expert_cache *c, int32_t layer, const int32_t *topk_ids,
                               int32_t T, int32_t k, int32_t *slot_of_expert,
                               hipStream_t compute_stream);

/*
 * ft_expert_cache_step_split -- the same LRU update and fills, but hits run
 * before the fills land (FreeToken 290b model page, "Cómo gestiona FreeToken
 * el prellenado y la decodificación": a hit runs on the GPU at once, a miss
 * is filled first).  Two slot tables (DEVICE, [E] each) replace
 * slot_of_expert: slot_hits gives the slot of every hit and FT_SLOT_SKIP for
 * the step's other needed experts; slot_misses gives the slot of every filled
 * miss, FT_SLOT_SKIP for the hits and -1 for misses left to the CPU; experts
 * not needed are -1 in both.  *n_filled (host, may be NULL) receives the
 * number of fills.  compute_stream is NOT made to wait for the fills:
 *
 *   step_split -> ft_moe_grouped_ffn(slot_hits, shared expert) ->
 *   ft_expert_cache_wait_fills -> ft_moe_grouped_ffn(slot_misses, no shared
 *   expert; only if *n_filled > 0) -> [CPU misses] -> ft_moe_combine
 *
 * The next step, resize or destroy still orders itself after the fills.
 * Errors as ft_expert_cache_step; slot_hits == slot_misses -> FT_EINVAL.
 */
ft_status ft_expert_cache_step_split(ft_expert_cache *c, int32_t layer, const int32_t *topk_ids, int32_t T, int32_t k,
                                     int32_t *slot_hits, int32_t *slot_misses, int32_t *n_filled,
                                     hipStream_t compute_stream);

/*
 * ft_expert_cache_plan + ft_expert_cache_fill -- ft_expert_cache_step_split in
 * two calls, so that the hits' FFN is queued before the host waits for the
 * LRU kernel (the same page and section: hits run at once).  plan validates,
 * makes compute_stream wait for an earlier layer prefetch's fills, enqueues
 * the LRU update writing slot_hits and slot_misses (as step_split) and
 * returns without waiting.  Between the two calls the caller may enqueue on
 * compute_stream work that reads slot_hits and the hit slots (not
 * slot_misses); fill (host) waits for the LRU kernel, enqueues the misses'
 * fills and writes their number to *n_filled (host, may be NULL):
 *
 *   plan -> ft_moe_grouped_ffn(slot_hits, shared expert) -> fill ->
 *   ft_expert_cache_wait_fills -> ft_moe_grouped_ffn(slot_misses) -> ...
 *
 * A plan must be followed by its fill before any other call that changes the
 * cache (step, step_split, plan, prefetch, resize, CPU-miss staging):
 * those return FT_EINVAL meanwhile, as does fill without a plan.  Errors of
 * the LRU update (FT_ECAPACITY, ids out of range) are returned by fill; the
 * cache state is then unchanged and the work queued since the plan read
 * tables that are not valid (discard its outputs).
 */
ft_status ft_expert_cache_plan(ft_expert_cache *c, int32_t layer, const int32_t *topk_ids, int32_t T, int32_t k,
                               int32_t *slot_hits, int32_t *slot_misses, hipStream_t compute_stream);
ft_status ft_expert_cache_fill(ft_expert_cache *c, int32_t *n_filled);

/* Makes compute_stream wait for the fills of the last split step (step_split or
 * plan + fill; a no-op when it had none or they were already waited for). */
ft_status ft_expert_cache_wait_fills(ft_expert_cache *c, hipStream_t compute_stream);

/* Totals since create (host).  */
ft_status ft_expert_cache_stats(const ft_expert_cache *c, ft_cache_stats *out);

/*
 * ft_expert_cache_set_trace -- keep an event log (for parity checks of the
 * cache's decisions against a simulator).  Off by default.  max_events > 0
 * allocates a ring of that many ft_cache_event records (host memory, here and
 * nowhere else) and empties it; once full, each new event overwrites the
 * oldest (counted in ft_cache_stats.trace_dropped).  0 turns the log off and
 * frees it.  Errors: max_events outside 0..2^28 or no memory -> FT_EINVAL.
 */
ft_status ft_expert_cache_set_trace(ft_expert_cache *c, int64_t max_events);

/* Copy the events the ring holds into host_buf (host) as ft_cache_event
 * records, oldest first, events of one step in ascending expert id.  *needed
 * (host, optional) receives the bytes they take; at most `bytes` are written
 * (whole records only).  Nothing is recorded while the log is off. */
ft_status ft_expert_cache_trace(const ft_expert_cache *c, void *host_buf, size_t bytes,
                                size_t *needed);

/* Current slot of (layer, expert) according to the host mirror of the last
 * completed step (-1 if not resident), written to *slot (host). */
ft_status ft_expert_cache_lookup(const ft_expert_cache *c, int32_t layer, int32_t expert,
                                 int32_t *slot);

/*
 * ft_expert_cache_set_split -- hybrid execution of misses (FreeToken 290b model
 * page, "Ejecución híbrida" and "Cómo gestiona FreeToken el prellenado y la
 * decodificación": misses are either filled over PCIe or run on the CPU, by a
 * split derived from two measured bandwidths).  From the next step on, of a
 * step's m misses only q are filled: the q in 0..m minimising
 * max(q / b_pcie, (m - q) / b_host), ties to the larger q (b_pcie: pinned
 * host-to-device expert bandwidth; b_host: bandwidth the host CPU expert
 * kernel achieves, both in the same unit); the lowest expert ids are filled.
 * The others stay non-resident (slot -1 in slot_of_expert, no eviction, no
 * recency; still counted as misses) and are listed by
 * ft_expert_cache_cpu_misses; ft_expert_cache_stage_cpu_misses and
 * ft_expert_cache_run_cpu_misses compute their rows on the host and write
 * them into y_rows after ft_moe_grouped_ffn (which writes NaN there).  b_host = 0 turns the split off (every miss filled, the default).
 * With b_host > 0 the host-mapped buffers of the CPU misses are allocated
 * here, for steps of up to T_max tokens with k picks each (a later call with
 * larger sizes replaces them); a stage call for a larger step returns
 * FT_ECAPACITY.  With b_host = 0, T_max and k are ignored.
 * Errors: negative or NaN bandwidths, or (b_host > 0) T_max < 1, k < 1 or
 * T_max*k > 2^28 -> FT_EINVAL; a planned step waiting for its fill ->
 * FT_EINVAL; FT_EHIP if the pinned allocation fails.
 */
ft_status ft_expert_cache_set_split(ft_expert_cache *c, double b_pcie, double b_host, int32_t T_max, int32_t k);

/* The last step's misses left to the CPU, ascending expert id: *n (host)
 * receives their number, experts (host) the first min(*n, capacity) ids. */
ft_status ft_expert_cache_cpu_misses(const ft_expert_cache *c, int32_t *experts, int32_t capacity,
                                     int32_t *n);

/*
 * Running the last step's CPU misses (FreeToken 290b model page, "Ejecución
 * híbrida"), in two calls around ft_moe_grouped_ffn on the compute stream:
 *
 *   ft_expert_cache_step -> ft_expert_cache_stage_cpu_misses ->
 *   ft_moe_grouped_ffn -> ft_expert_cache_run_cpu_misses -> ft_moe_combine
 *
 * stage: enqueues on `stream` a kernel that copies x [T, H] (DEVICE, bf16,
 *   16-byte aligned), expert_offsets [E+1] and sorted_rows [T*k] (DEVICE, the
 *   step's ft_moe_permute outputs) into host-mapped memory the cache owns
 *   (sized by ft_expert_cache_set_split).  A kernel, not a DMA copy: it does
 *   not wait behind the step's miss fills on the copy engines.  Returns at
 *   once, after waiting for the previous stage's kernel if it is still queued.
 * run: waits for that kernel only, computes the rows of every CPU miss on the
 *   host (ft_cpu_miss_rows over the cache's host bank, n_threads as there),
 *   then enqueues on `stream` a kernel that copies them from host-mapped
 *   memory into y_rows [T*k, H] (DEVICE, fp32, 16-byte aligned), replacing
 *   the NaN rows ft_moe_grouped_ffn left there; enqueue it after that FFN.
 * Both are no-ops (FT_OK) when the last step left no miss to the CPU.
 * Errors: run without a stage of the same step -> FT_EINVAL; activations
 *   other than bf16 -> FT_ENOTSUP; a step larger than set_split's T_max x k
 *   -> FT_ECAPACITY (stage); the host kernel's errors as there.
 * A later stage or run waits for the previous one's kernels before it reuses
 * the host buffers.
 */
ft_status ft_expert_cache_stage_cpu_misses(ft_expert_cache *c, const void *x, int32_t x_dtype, int32_t T, int32_t k,
                                           const int32_t *expert_offsets, const int32_t *sorted_rows,
                                           hipStream_t stream);
ft_status ft_expert_cache_run_cpu_misses(ft_expert_cache *c, float *y_rows, hipStream_t stream, int32_t n_threads);

/*
 * ft_expert_cache_prefetch_layer -- bring every expert of `layer` into the
 * cache ahead of its step: full-layer double buffering in prefill (while the
 * GPU computes one layer, the next layer's experts stream over PCIe, when the
 * cache has room: FreeToken linux page, "Cómo gestiona FreeToken la memoria
 * MoE"; FreeToken 290b model page, "Cómo gestiona FreeToken el prellenado y la
 * decodificación"; the same cache serves prefill and decode).  The LRU is
 * updated as by a step of `layer` whose routing uses all E experts, but the
 * prefetch is not a routed access: it adds fills, bytes and evictions, not
 * accesses, hits or misses.  The LRU kernel runs on compute_stream (the host
 * waits for it, as in a step); the fills go to the copy queues and are NOT
 * waited for here: the next ft_expert_cache_step makes its compute stream
 * (and its own fills) wait for them.  Intended order per layer l: step(l),
 * prefetch(l+1), then the FFN of layer l.  The pages double-buffer only when
 * the cache has room: the prefetch never takes the slot of an entry the most
 * recent step (step, step_split or plan + fill) left resident for its
 * routing, so the FFN of layer l still reads its own experts; the layer's
 * experts are visited in ascending id, and once no other slot is left the
 * rest are not prefetched (event code 5) and miss in their own step.  With
 * room for two layers every expert is prefetched.
 * Errors: E > capacity -> FT_ECAPACITY (cache unchanged); as for a step.
 */
ft_status ft_expert_cache_prefetch_layer(ft_expert_cache *c, int32_t layer, hipStream_t compute_stream);

/*
 * ft_expert_cache_resize -- change the number of slots at a safe point (the
 * runtime resizes and rebuilds the GPU expert cache at safe points of its
 * scheduler when the GPU memory budget changes: FreeToken quantization page,
 * "Flujo de configuración de la cuantización de FreeToken"; FreeToken 290b
 * model page, "Caché elástica").  The min(new_capacity, resident) most
 * recently used entries are kept and compacted into slots 0.. in ascending
 * order of their old slot; the others are dropped (counted as evictions);
 * recency and later decisions continue as if the cache had always had the
 * kept entries in those slots.  Kept blobs are copied into new_slot_pool
 * (device, new_capacity * expert_bytes, caller-owned; it may be the current
 * pool when that allocation holds new_capacity slots -- entries only move to
 * lower slots, so the copies are safe in place).  The cache borrows
 * new_slot_pool from then on.  The call waits for `stream` (the stream the
 * cache steps run on) and the copy stream, and returns when the new state
 * and the copies are complete: a rare call, not for the per-token path.
 * Errors: new_capacity < 1 or a non-device pool -> FT_EINVAL; above 65536
 * slots -> FT_ENOTSUP; on FT_EHIP the cache is unchanged.
 */
ft_status ft_expert_cache_resize(ft_expert_cache *c, int32_t new_capacity, void *new_slot_pool,
                                 hipStream_t stream);

/* Free the cache's own state.  Waits for its pending copies first. */
ft_status ft_expert_cache_destroy(ft_expert_cache *c);

/* ------------------------------------------------------------------------ */
/* Workspace sizes                                                            */
/* ------------------------------------------------------------------------ */
enum { FT_WS_PERMUTE = 1, FT_WS_FFN = 2, FT_WS_ROUTE_PERMUTE = 3, FT_WS_LAYER = 4 };

/* Bytes of workspace the call `which` needs for these sizes (0 if none).
 * For FT_WS_FFN, H and I are those of the layout and the shared expert is
 * assumed present (an upper bound either way). */
size_t ft_workspace_bytes(int32_t which, int32_t T, int32_t k, int32_t E, int32_t H, int32_t I);

#ifdef __cplusplus
}
#endif
#endif /* FT_MOE_H */
