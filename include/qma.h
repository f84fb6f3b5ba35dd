/*
 * qma.h -- C ABI of libqma, an MI355X (gfx950) library for the W4A16 MoE
 * expert GEMM pair: gate_up, then a gated activation, then down.
 * Weights are uint4 with group-32 bf16 scales; activations are bf16.
 *
 * Sources. The operation is the one described in two pages:
 *   [release]  "vLLM and Novita AI release Chord: a fast INT4 MoE kernel for
 *              Kimi K2.x" (agentlenshq.com, Japanese);
 *   [announce] "vLLM announces that the Humming backend can run Novita's
 *              open-source Chord kernel" (arex-research.com, Chinese).
 *
 * Conventions for every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller. Tensors are
 *     contiguous and row-major, and 16-byte aligned unless a call says
 *     otherwise. The library never frees or retains them past the call.
 *   - bf16 values are passed as uint16_t bit patterns; indices are int32.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     GPU calls only enqueue work on it. None synchronises with the host
 *     except qma_validate_routing, and none allocates device memory (a
 *     workspace is passed in where one is needed). The trusted forward
 *     path is therefore capturable in a hipGraph ([release] runtime
 *     considerations: capturable when routing validation is off).
 *   - Every call returns a qma_status and never aborts. On failure,
 *     qma_last_error_detail() returns text for the calling thread.
 *   - Host objects (qma_layer_t, qma_plan_t) are immutable once created
 *     and may be shared between threads.
 */
#ifndef QMA_H
#define QMA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qma_status {
  QMA_OK = 0,
  QMA_ERR_INVALID_ARG = 1,   /* null pointer, bad shape, short capacity */
  QMA_ERR_UNSUPPORTED = 2,   /* quantisation scheme this library rejects */
  QMA_ERR_ROUTING = 3,       /* routing buffers fail validation */
  QMA_ERR_WORKSPACE = 4,     /* workspace missing or too small */
  QMA_ERR_HIP = 5            /* a HIP runtime call or launch failed */
} qma_status;

/* The three families of GEMM call ([announce] scheduling section: the
 * indexed path consumes vLLM's routing tensors; grouped_contiguous
 * (prefill) and grouped_masked (decode) form a separate family with their
 * own routing convention). */
typedef enum qma_path {
  QMA_PATH_INDEXED = 0,
  QMA_PATH_GROUPED_CONTIGUOUS = 1,
  QMA_PATH_GROUPED_MASKED = 2
} qma_path;

enum { QMA_DTYPE_BF16 = 1, QMA_DTYPE_FP16 = 2, QMA_DTYPE_FP32 = 3 };
/* 8 uint4 values per int32 word along K; element k % 8 at bits 4*(k%8).. */
enum { QMA_PACK_INT32_K8 = 1 };

/* Quantisation scheme of a projection ([announce] integration section: the
 * schema supports uint4, group 32 and BF16 scales; other schemes fail at
 * load instead of falling back). The only accepted value is
 * {4, 8, 32, QMA_DTYPE_BF16, QMA_DTYPE_BF16, QMA_PACK_INT32_K8}. */
typedef struct qma_quant_desc {
  int32_t weight_bits;   /* 4 */
  int32_t zero_point;    /* 8: w = (q - 8) * scale */
  int32_t group_size;    /* 32 elements of K per scale */
  int32_t scale_dtype;   /* QMA_DTYPE_BF16 */
  int32_t act_dtype;     /* QMA_DTYPE_BF16 */
  int32_t pack_format;   /* QMA_PACK_INT32_K8 */
} qma_quant_desc;

/* Profile inferred from the projection's shape alone, with no shard
 * arguments ([release] runtime considerations). EP shares hold a few
 * experts with large N*K each; TP shares hold many experts with N or K cut
 * by the tensor-parallel degree. */
typedef enum qma_profile {
  QMA_PROFILE_GENERIC = 0,
  QMA_PROFILE_EP_GATE_UP = 1,
  QMA_PROFILE_EP_DOWN = 2,
  QMA_PROFILE_TP_GATE_UP = 3,
  QMA_PROFILE_TP_DOWN = 4
} qma_profile;

typedef struct qma_layer qma_layer_t;

/* GEMM kernel families the planner chooses between. */
typedef enum qma_kernel {
  /* Few rows per expert (decode, up to 79): 16-, 32- or 64-row token
   * tiles on the MFMA row side and weight columns on the column side, one
   * 16x16x32 MFMA per scale group. (The pages' decode kernel swaps the
   * operands because its MMA is 16 x 8, [announce] scheduling section; the
   * 16 x 16 shapes of CDNA4 need no swap.) HBM-bound; takes split-K. */
  QMA_KERNEL_SMALL_M = 1,
  /* Many rows per expert (prefill): token tiles staged in LDS, weights
   * dequantised into the MFMA column side. MFMA-bound. Every wave loads,
   * dequantises and multiplies; takes split-K. */
  QMA_KERNEL_LARGE_M = 2,
  /* Many rows per expert, producer/consumer form ([release] performance
   * highlights: a persistent main loop whose loads and dequantisation run
   * in dedicated warps beside the matrix operations): a persistent grid
   * of one workgroup per compute unit in which producer waves stage token
   * rows and dequantised weights in LDS and consumer waves only run MFMAs.
   * Same 128 x 256 blocks and bit-identical results as
   * QMA_KERNEL_LARGE_M; no split-K. Never chosen by the planner (it runs
   * slower than QMA_KERNEL_LARGE_M on gfx950); a caller selects it by
   * setting plan.kernel. */
  QMA_KERNEL_LARGE_M_PC = 3
} qma_kernel;

/* A plan: a pure function of the layer's shape and the host-known token
 * counts ([announce] scheduling section: the schedule follows the routed
 * tokens per expert, not the total; profile and layout are fixed at load
 * and the token count only tunes the schedule within them). Every field is
 * plain data so tests can check the rules. A caller may edit kernel,
 * block_m, block_n, split_k, k_depth, waves_k, n_stream and schedule; the
 * GEMM calls validate the plan against the layer and reject, with
 * QMA_ERR_INVALID_ARG and before any launch, a plan made for another layer
 * or one that names no compiled kernel instance, or whose split_k is
 * outside [1, 8] or above K/128 (every K partition owns at least one
 * 128-wide chunk). Compiled instances: small-M with block_m in {16, 32, 64}
 * and waves_k in {1, 2, 4}, where a wave owns block_n / (16 * 4 / waves_k)
 * 16-column tiles (1, 2 or 4) and block_m / 16 row tiles; waves_k = 1 with
 * 2 or 4 column tiles takes up to 8 (row x column) tiles per wave, every
 * other small-M shape up to 4; large-M: a 128 x 256 block, and split_k = 1
 * for the producer/consumer form. k_depth
 * outside an instance's supported depths falls back to that instance's
 * default. */
typedef struct qma_plan {
  int32_t path;          /* qma_path of the layer */
  int32_t kernel;        /* qma_kernel */
  int32_t block_m;       /* rows per routing block (the moe_align block size) */
  int32_t block_n;       /* output columns per workgroup */
  int32_t split_k;       /* K partitions across workgroups; 1 = off */
  int32_t k_depth;       /* K elements in flight per wave */
  int32_t num_experts;   /* E of the layer */
  int32_t n;             /* N of the layer */
  int32_t k;             /* K of the layer */
  int32_t rows;          /* rows planned for: T*topk, M, or E*budget */
  int32_t tok_e_x100;    /* routed rows per expert x 100, host estimate */
  int32_t est_tiles;     /* M x N tiles expected without split-K; the launch also
                            spreads few token tiles over the XCDs from it */
  int32_t profile;       /* qma_profile */
  int32_t waves_k;       /* K partitions inside one workgroup */
  int32_t expected_m;    /* masked layers: the expected_m planned for, else 0 */
  int32_t n_stream;      /* N blocks one workgroup streams through (>= 1) */
  int32_t schedule;      /* QMA_SCHEDULE_*: how (tile, column block) work is handed out */
} qma_plan_t;

/* How a small-M GEMM hands out its (token tile, column block) work
 * ([announce] scheduling section: semi-static token-slice scheduling
 * against dynamic scheduling at 9..15 tokens per expert).
 *   SEMI_STATIC: the grid is sized from host-known shapes and each
 *     workgroup derives its tile, expert and rows from the routing buffers
 *     on the device; workgroups past num_tokens_padded exit at once. The
 *     planner's default, except where it picks GANG.
 *   DYNAMIC: a persistent grid (three workgroups per CU) whose workgroups
 *     take items from a device work counter until the routed items run
 *     out. The counter lives in the workspace (qma_workspace_bytes counts
 *     it) and is reset by a one-thread kernel on the same stream before the
 *     GEMM. Only 16/32-row tiles with one K partition, no split-K and
 *     n_stream = 1 accept it; other plans -> QMA_ERR_INVALID_ARG.
 *   GANG: the semi-static item order, run by one workgroup per CU holding
 *     three groups of four waves, each group on its own (tile, column
 *     block, split) item. The groups share one barrier per K chunk, so the
 *     items on a CU advance together and end together, where separate
 *     workgroups would end staggered and leave the CU streaming with few
 *     loads in flight. Items beyond one round loop in the same order. The
 *     planner picks it for shared-row plans with one K partition and at
 *     least 8 K chunks whose items fill one such round: at least 5/6 of the
 *     3 x 256 slots, and at most the 3 x 32 slots of an XCD on the fullest
 *     XCD (token tiles are dealt to the 8 XCDs in turn), trying the plan's
 *     width, then 256, then 128 columns. Accepted for waves_k = 1,
 *     n_stream = 1, block_n 128 or 256 and block_m 16, 32 or 64 (the
 *     shared-row instances), with or without split-K; other plans ->
 *     QMA_ERR_INVALID_ARG. No workspace beyond split-K's.
 *   STREAM_K: the gang's one workgroup per CU, for launches of several
 *     rounds. Each CU takes a contiguous share of the (token tile, column
 *     block) items, balanced to one item, and its groups split the share's
 *     K chunks evenly, so an item may be cut in K between neighbouring
 *     groups of a CU ([release] indexed techniques: stream-K). The pieces
 *     meet in LDS and are added in K order, so the result is that of
 *     split-K over the same cut points: with integer-exact inputs, bit for
 *     bit the unsplit result. Accepted on the INDEXED path for waves_k = 1, n_stream = 1,
 *     split_k = 1, block_m 16 or 32, block_n 128 or 256 and at least 8 K
 *     chunks; other plans -> QMA_ERR_INVALID_ARG. A call whose sorted
 *     capacity could give one group items of three token tiles (column
 *     blocks per tile fewer than the items per group) -> QMA_ERR_INVALID_ARG.
 *     No workspace. The planner does not pick it: on the measured shapes
 *     the gang and semi-static schedules were as fast or faster. */
typedef enum {
  QMA_SCHEDULE_SEMI_STATIC = 0,
  QMA_SCHEDULE_DYNAMIC = 1,
  QMA_SCHEDULE_GANG = 2,
  QMA_SCHEDULE_STREAM_K = 3
} qma_schedule;

/* ---- layer (load time) ------------------------------------------------ */

/* Checks the scheme and fixes the profile and the packed layout from
 * (E, N, K) ([release] runtime considerations; [announce] scheduling and
 * integration sections). N is the output width, K the reduction length.
 * Errors: any scheme other than the accepted one -> QMA_ERR_UNSUPPORTED;
 * E < 1, N % 16 != 0, K % 128 != 0, N or K < 1, a null pointer ->
 * QMA_ERR_INVALID_ARG. K must be a multiple of 128, not only of the scale
 * group (32): the packed layout is built from 128-wide K chunks, and every
 * projection of the pages' models has such a K (7168, 2048, 256). The
 * caller owns *out and frees it with qma_layer_destroy. */
qma_status qma_layer_create(const qma_quant_desc* q, int32_t E, int32_t N,
                            int32_t K, qma_path path, qma_layer_t** out);

/* Layer flags for qma_layer_create_ex. */
typedef enum {
  /* A gate_up layer with the gated activation fused into its GEMMs
   * ([announce] measurement section: an activation, silu(gate) * up, sits
   * between gate_up and down). The checkpoint has N = 2I rows: gate rows
   * [0, I), then up rows [I, 2I). The GEMMs of such a layer write
   * h = silu(gate) * up, [rows, I] bf16 with row stride I, instead of the
   * [rows, 2I] gate_up output; gate and up are each rounded to bf16 first,
   * as the unfused GEMM stores them, so h equals qma_silu_and_mul on the
   * unfused output bit for bit. The packed layout pairs gate tile q with up
   * tile q (qma_prepack writes it). Needs N % 64 == 0; a plan must give each
   * wave an even number of 16-column tiles (every planner plan does) and
   * must not name QMA_KERNEL_LARGE_M_PC -> QMA_ERR_INVALID_ARG. Split-K
   * partials stay in the packed column order and the reduction applies the
   * activation. */
  QMA_LAYER_FUSE_SILU_MUL = 1
} qma_layer_flag;

/* qma_layer_create with flags (qma_layer_flag bits; 0 is qma_layer_create).
 * Unknown bits -> QMA_ERR_INVALID_ARG. */
qma_status qma_layer_create_ex(const qma_quant_desc* q, int32_t E, int32_t N, int32_t K,
                               qma_path path, uint32_t flags, qma_layer_t** out);
void qma_layer_destroy(qma_layer_t* layer);
/* Reads back the shape, path and inferred profile. Null outputs are
 * skipped. */
qma_status qma_layer_info(const qma_layer_t* layer, int32_t* E, int32_t* N,
                          int32_t* K, int32_t* path, int32_t* profile);

/* Bytes of the packed weight buffer qma_prepack writes (weights + scales). */
size_t qma_packed_weight_bytes(const qma_layer_t* layer);

/* Load-time conversion of the checkpoint layout into the library's tiled
 * layout ([announce] scheduling section: the weight layout is fixed when
 * the model loads; [release] grouped techniques: weights packed in
 * BLOCK_K = 128 chunks).
 *   qweight [E, N, K/8] int32: 8 uint4 per word along K, nibble k%8 at bits
 *           4*(k%8)..+3 (compressed-tensors pack-quantized INT4 group 32)
 *   scales  [E, N, K/32] bf16
 *   packed  qma_packed_weight_bytes(layer) bytes, 256-byte aligned
 * All three are device buffers. The inputs are read and not kept. Errors:
 * a null or misaligned pointer -> QMA_ERR_INVALID_ARG. */
qma_status qma_prepack(const qma_layer_t* layer, const int32_t* qweight,
                       const uint16_t* scales, void* packed, void* stream);

/* ---- planning (host only) --------------------------------------------- */

/* Plan the indexed GEMM for T tokens routed top-`topk` over the layer's E
 * experts. tok_e = T*topk/E picks block_m ([release] indexed techniques: a
 * block-M heuristic keyed on routed tokens per expert, switching at 80),
 * block_n comes from the tile count ([release] grouped techniques: the
 * wider tile only when enough N tiles exist, never below 128 columns with
 * long K), and split-K turns on only when the grid would hold fewer than
 * two workgroups per compute unit ([release] indexed techniques: the
 * stream-K gate); it then aims at three per compute unit and keeps at
 * least 14 K chunks of 128 per split. An underfilled grid whose K is too
 * short to split takes 64-column blocks with the waves on K (waves_k = 4)
 * instead. Plans whose items fill one round of the gang
 * schedule take it (QMA_SCHEDULE_GANG, with its width rule); the others
 * are semi-static. force_block_m = 0 lets the planner choose;
 * otherwise 16, 32 or 64 selects the small-M kernel with that tile and 128
 * the large-M kernel (which needs N % 256 == 0). The down projection passes
 * gate_up's block_m so one moe_align serves both. Errors: T < 0, topk < 1,
 * a force_block_m outside {0,16,32,64,128}, 128 with N % 256 != 0, or a
 * layer whose path is not INDEXED -> QMA_ERR_INVALID_ARG. */
qma_status qma_plan_indexed(const qma_layer_t* layer, int32_t T, int32_t topk,
                            int32_t force_block_m, qma_plan_t* out);

/* Plan a grouped GEMM. Contiguous layers: m_rows_or_budget = M, the padded
 * row count (a multiple of 128), and expected_m is ignored; the large-M
 * kernel is used whenever N % 256 == 0, since each 128-row tile belongs to
 * one expert ([release] grouped techniques: contiguous prefill pads each
 * expert to a 128-row boundary).
 * Masked layers:
 * m_rows_or_budget = the per-expert row budget, and expected_m = the
 * host-side estimate of valid rows that picks block_m ([release] grouped
 * techniques: BLOCK_M from the expected token count). */
qma_status qma_plan_grouped(const qma_layer_t* layer, int32_t m_rows_or_budget,
                            int32_t expected_m, qma_plan_t* out);

/* Bytes of workspace the plan's GEMM needs: the fp32 split-K partials when
 * split is on, plus 256 bytes for the work counter of a DYNAMIC schedule
 * (0 for a semi-static plan without split). */
size_t qma_workspace_bytes(const qma_plan_t* plan);

/* ---- routing ---------------------------------------------------------- */

/* Capacities that always suffice for moe_align:
 *   sorted_cap = T*topk + E*(block_m - 1);  blocks_cap = ceil(sorted_cap / block_m).
 * Errors: negative T, topk < 1, E < 1, block_m < 1 -> QMA_ERR_INVALID_ARG. */
qma_status qma_align_sizes(int32_t T, int32_t topk, int32_t E, int32_t block_m,
                           int32_t* sorted_cap, int32_t* blocks_cap);

/* Block-aligned routing buffers ([announce] scheduling section: the
 * indexed path consumes sorted_ids / expert_ids / num_tokens_padded;
 * [release] runtime considerations: over-allocated buffers).
 * topk_ids [T, topk] int32 names each slot's expert; slot i = t*topk + k.
 * Ids outside [0, E) mean "not on this rank" and are left out. Outputs:
 *   sorted_ids [sorted_cap]: expert by expert in ascending order, the
 *     expert's slots in ascending order, padded with the sentinel T*topk up
 *     to a multiple of block_m; every entry past num_tokens_padded is the
 *     sentinel;
 *   expert_ids [ceil(sorted_cap/block_m)]: the expert of each block, -1
 *     past the last;
 *   num_tokens_padded [1]: the padded length.
 * An expert with no slots gets no block. The result is deterministic
 * (bit-exact). Errors: sorted_cap below the qma_align_sizes bound,
 * E > 1024, T*topk >= 2^31 - E*block_m, or a null pointer ->
 * QMA_ERR_INVALID_ARG. */
qma_status qma_moe_align(const int32_t* topk_ids, int32_t T, int32_t topk,
                         int32_t E, int32_t block_m, int32_t* sorted_ids,
                         int32_t* expert_ids, int32_t* num_tokens_padded,
                         int32_t sorted_cap, void* stream);

/* Routing validation, the opt-in check the trusted path skips ([release]
 * runtime considerations). Reads the buffers back: it SYNCHRONISES the
 * stream and is not capturable. It checks that every id is in [-1, E),
 * recomputes on the host the buffers qma_moe_align defines for topk_ids,
 * and compares all of them over the whole capacity: num_tokens_padded,
 * sorted_ids [sorted_cap] (slot order inside each segment, the sentinel in
 * every padding position and in the tail) and expert_ids
 * [ceil(sorted_cap/block_m)] (routed blocks and the -1 tail). It returns
 * QMA_ERR_ROUTING on the first difference, with text naming the position.
 * Errors: negative sizes or a null buffer -> QMA_ERR_INVALID_ARG. */
qma_status qma_validate_routing(const int32_t* topk_ids, int32_t T,
                                int32_t topk, int32_t E, int32_t block_m,
                                const int32_t* sorted_ids,
                                const int32_t* expert_ids,
                                const int32_t* num_tokens_padded,
                                int32_t sorted_cap, void* stream);

/* Checks a contiguous layout: every aligned 128-row block of m_indices
 * [M] holds one expert id, then only -1, and ids are < E. Synchronises.
 * Returns QMA_ERR_ROUTING on a violation. */
qma_status qma_validate_contiguous(const int32_t* m_indices, int32_t M,
                                   int32_t E, void* stream);

/* ---- GEMMs ------------------------------------------------------------ */

/* Indexed expert GEMM ([announce] scheduling section; [release] indexed
 * techniques). For every block b < *num_tokens_padded / block_m with
 * expert e = expert_ids[b], and every row s = sorted_ids[b*block_m + i]
 * with s < num_slots:
 *   c[s, n] = bf16( sum_k a[s / a_row_div, k] * (q_e[n,k] - 8) * scale_e[n, k/32] )
 *             (times topk_weights[s] when topk_weights is not NULL)
 * with fp32 accumulation. gate_up passes a_row_div = topk (the token's
 * row); down passes 1 (the slot's own row of the activation output).
 *   a        [a_rows, K] bf16
 *   packed_w the layer's prepacked weights
 *   routing  buffers from qma_moe_align with block_m = plan->block_m;
 *            only device memory is read (no host sync), so the buffers may
 *            be over-allocated up to sorted_cap
 *   c        [num_slots, N] bf16; rows no block names are left untouched
 *   ws       qma_workspace_bytes(plan) bytes of device memory, or NULL if 0
 * Errors: a plan made for another layer shape or path, a null pointer, or
 * a sorted_cap below num_slots + E*(block_m - 1) (the qma_align_sizes
 * bound) -> QMA_ERR_INVALID_ARG; a short workspace -> QMA_ERR_WORKSPACE. */
qma_status qma_indexed_gemm(const qma_layer_t* layer, const qma_plan_t* plan,
                            const uint16_t* a, int32_t a_rows,
                            int32_t a_row_div, const void* packed_w,
                            const int32_t* sorted_ids,
                            const int32_t* expert_ids,
                            const int32_t* num_tokens_padded,
                            int32_t sorted_cap, int32_t num_slots,
                            const float* topk_weights, uint16_t* c, void* ws,
                            size_t ws_bytes, void* stream);

/* qma_indexed_gemm for callers that cannot allocate device memory: code
 * under hipGraph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments, results and errors as qma_indexed_gemm, minus
 * the workspace: a plan that needs one (split-K partials, the dynamic
 * schedule's counter) uses the library's static device scratch, a fixed
 * 32 MiB array that every device the library runs on holds until the
 * process ends. A plan needing more than 32 MiB (qma_workspace_bytes) ->
 * QMA_ERR_WORKSPACE before any launch. The call allocates nothing; the
 * first call on a device looks up that device's scratch address. All calls
 * on one device share its scratch, and the scratch keeps the last call's
 * contents (the kernels write every partial they read and reset the
 * counter themselves): calls that overlap on one device, on different
 * streams or threads, race on it and must be serialised by the caller. */
qma_status qma_indexed_gemm_scratch(const qma_layer_t* layer, const qma_plan_t* plan,
                                    const uint16_t* a, int32_t a_rows,
                                    int32_t a_row_div, const void* packed_w,
                                    const int32_t* sorted_ids,
                                    const int32_t* expert_ids,
                                    const int32_t* num_tokens_padded,
                                    int32_t sorted_cap, int32_t num_slots,
                                    const float* topk_weights, uint16_t* c,
                                    void* stream);

/* Grouped contiguous GEMM ([release] grouped techniques: contiguous
 * prefill pads each expert to 128 rows). c[r] = a[r] . W[m_indices[r]]^T
 * for rows with m_indices[r] >= 0.
 *   a [M, K], m_indices [M] (device; -1 = padding), c [M, N];
 *   M % 128 == 0. Padding rows of c are left untouched, and padding rows
 *   of a are never read.
 * The one-expert-per-128-row-block convention is checked only by
 * qma_validate_contiguous. A row whose id differs from its block's first
 * row is treated as padding. */
qma_status qma_grouped_contiguous_gemm(const qma_layer_t* layer,
                                       const qma_plan_t* plan,
                                       const uint16_t* a,
                                       const int32_t* m_indices, int32_t M,
                                       const void* packed_w, uint16_t* c,
                                       void* ws, size_t ws_bytes,
                                       void* stream);

/* Grouped masked GEMM ([release] grouped techniques: masked decode keeps
 * a fixed row budget per expert). c[e, r] = a[e, r] . W[e]^T for
 * r < masked_m[e].
 *   a [E, Mb, K]; masked_m [E] is device memory, with values clamped to
 *   [0, Mb]; c [E, Mb, N]. expected_m must equal the plan's.
 * Rows r >= masked_m[e] are neither read nor written. */
qma_status qma_grouped_masked_gemm(const qma_layer_t* layer,
                                   const qma_plan_t* plan, const uint16_t* a,
                                   const int32_t* masked_m, int32_t Mb,
                                   int32_t expected_m, const void* packed_w,
                                   uint16_t* c, void* ws, size_t ws_bytes,
                                   void* stream);

/* ---- router --------------------------------------------------------- */

/* The router step before moe_align: each token goes to its top-k experts
 * (the pages' scenarios route tokens top-k over the layer's experts,
 * [announce] measurement section; [release] performance highlights).
 * For token t, topk_ids[t, 0..topk) are the experts with the largest
 * logits, best first, equal logits going to the lower expert index, and
 * topk_weights[t, i] is that expert's softmax probability over all E
 * experts (not renormalised over the chosen k).
 *   logits       [T, E] float32, finite values (others: unspecified result)
 *   topk_ids     [T, topk] int32 out
 *   topk_weights [T, topk] float32 out (may be NULL)
 * All device buffers, 4-byte aligned. Errors: T < 0, E outside [1, 1024],
 * topk outside [1, min(E, 16)], a null required buffer ->
 * QMA_ERR_INVALID_ARG. */
qma_status qma_router_topk(const float* logits, int32_t T, int32_t E,
                           int32_t topk, int32_t* topk_ids,
                           float* topk_weights, void* stream);

/* ---- activation and combine ------------------------------------------- */

/* The gated activation between gate_up and down ([announce] measurement
 * section names an activation between the two GEMMs; the gate is SiLU):
 *   y[r, j] = bf16( silu(x[r, j]) * x[r, I + j] ), computed in fp32.
 *   x [R, 2I] bf16 (gate half first), y [R, I] bf16.
 * Errors: R < 0, I < 1, or a null pointer -> QMA_ERR_INVALID_ARG. */
qma_status qma_silu_and_mul(const uint16_t* x, uint16_t* y, int64_t R,
                            int32_t I, void* stream);

/* Top-k combine after down (the step the pages leave out of the kernel
 * timing): out[t, n] = bf16( sum_k w[t,k] * c2[t*topk + k, n] ), with fp32
 * sums in k order. Slots whose expert id is outside [0, E) (NOT on this
 * rank) are skipped when topk_ids is given.
 *   c2 [T*topk, N] bf16, w [T, topk] fp32, topk_ids [T, topk] or NULL,
 *   out [T, N] bf16. */
qma_status qma_moe_combine(const uint16_t* c2, const float* w,
                           const int32_t* topk_ids, int32_t E, int32_t T,
                           int32_t topk, int32_t N, uint16_t* out,
                           void* stream);

/* ---- misc ------------------------------------------------------------- */

const char* qma_status_str(qma_status s);
/* Text of the last error on the calling thread ("" if none). */
const char* qma_last_error_detail(void);
/* Library version string. */
const char* qma_version(void);

#ifdef __cplusplus
}
#endif
#endif /* QMA_H */
