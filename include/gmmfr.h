/*
 * gmmfr -- fused quantized MoE grouped matmul with finalize-routing combine,
 * for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * Operation ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", CANN operator
 * documentation, function description): a GroupedMatmul whose output rows
 * are combined by index (MoeFinalizeRouting), in one call.
 *
 *   Rows of x1 (m,k) int8 are sorted by expert and split into e groups by
 *   groupList.  Row i of group g is multiplied by x2[g] (k,n) with int32
 *   accumulation:   acc[i][j] = sum_kk x1[i][kk] * x2[g][kk][j].
 *   It is dequantised and weighted, each product rounded to fp32:
 *       y[i][j] = ((float(acc[i][j]) * scale[g][0][j]) * pertokenScale[i]) * logit[i]
 *   (the order (acc * deqScale) * perTokenScale is the one spelled out by
 *   the worked example of "matmul支持pertoken量化模式", ATB per-token quant
 *   linear; the routing weight is applied last).
 *   MxA8W4 mode ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", Atlas 350
 *   notes on MxA8W4 quantisation): x1 FP8 E4M3, x2 FP4 E2M1 given as (e,n,k),
 *   and one E8M0 block scale per 32 k for each row of x1 (pertokenScale) and
 *   each weight column (scale):
 *       acc[i][j] = sum_b 2^(pts[i][b]-127) * 2^(scale[g][j][b]-127) * sum_{kk in b} x1[i][kk] * x2[g][j][kk]
 *   accumulated in fp32 by the matrix core (order unspecified), then
 *       y[i][j] = acc[i][j] * logit[i].
 *   FP8 mode (x1 and x2 FLOAT8_E4M3FN, x2 (e,k,n), or (e,n,k) when
 *   transposed): acc is the fp32
 *   sum of the FP8 products (order unspecified), then y as in the int8 mode:
 *       y[i][j] = ((acc[i][j] * scale[g][0][j]) * pertokenScale[i]) * logit[i].
 *   The output out (outputBS,n) fp32 starts at +0.0 with rows
 *   [sharedInputOffset, sharedInputOffset + bsdp) set to the widened bf16
 *   sharedInput, and every covered row i is added into out[rowIndex[i]].
 *
 * Two-stage use ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", interface
 * description: a first call validates and sizes the workspace, a second call
 * runs on a stream):
 *     size_t ws;  gmm_finalize_routing_workspace(&args, &ws);
 *     ... allocate ws bytes of device memory ...
 *     gmm_finalize_routing(&args, workspace, ws, stream);
 *
 * Ownership: every buffer, the workspace included, belongs to the caller and
 * is device memory (except tuning_config, a host array read during the call).
 * The library allocates and frees nothing, keeps no state between calls and
 * is safe to call from several host threads.  gmm_finalize_routing only
 * enqueues work on `stream` and returns; the caller keeps all buffers alive
 * until the stream passes that point.
 */
#ifndef GMMFR_H
#define GMMFR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ status codes
 * The first call validates the arguments and reports the first rule broken
 * ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", return value of the first
 * stage: errors are raised on invalid inputs).  Nothing is enqueued when a
 * call returns a non-zero status. */
typedef enum {
  GMMFR_OK = 0,
  GMMFR_ERR_NULLPTR = 1,      /* a required tensor, args or out-pointer is NULL   */
  GMMFR_ERR_DTYPE = 2,        /* element type not accepted for that tensor        */
  GMMFR_ERR_SHAPE = 3,        /* ranks or sizes inconsistent, or outside limits   */
  GMMFR_ERR_ATTR = 4,         /* groupListType, offsets, transposes, flags        */
  GMMFR_ERR_UNSUPPORTED = 5,  /* bias / offset / antiquant given, INT64 scale     */
  GMMFR_ERR_ALIGN = 6,        /* a base pointer is not 16-byte aligned            */
  GMMFR_ERR_WORKSPACE = 7,    /* workspace missing or smaller than required       */
  GMMFR_ERR_HIP = 8           /* the HIP runtime refused a launch                 */
} gmmfr_status;

/* ------------------------------------------------------------ element types */
typedef enum {
  GMMFR_DT_NONE = 0,
  GMMFR_DT_INT8 = 1,
  GMMFR_DT_INT4 = 2,     /* signed 4-bit, two per byte, low nibble = lower column */
  GMMFR_DT_INT32 = 3,
  GMMFR_DT_INT64 = 4,
  GMMFR_DT_FLOAT32 = 5,
  GMMFR_DT_BFLOAT16 = 6,
  GMMFR_DT_FLOAT8_E4M3FN = 7,  /* 1 sign, 4 exponent (bias 7), 3 mantissa; no inf; 0x7F/0xFF NaN */
  GMMFR_DT_FLOAT4_E2M1X2 = 8,  /* two FP4 E2M1 per byte, low nibble first (values 0,.5,1,1.5,2,3,4,6 and negatives) */
  GMMFR_DT_FLOAT8_E8M0 = 9     /* power-of-two scale 2^(b-127) per byte; 255 NaN */
} gmmfr_dtype;

/* A dense, row-major, contiguous device tensor.  data == NULL means "absent",
 * unless a dimension is 0 (an empty tensor may have a null pointer). */
typedef struct {
  void* data;
  int32_t dtype;      /* gmmfr_dtype */
  int32_t ndim;       /* 1..4        */
  int64_t dims[4];
} gmmfr_tensor;

/* Combine strategy (our addition; the operator is non-deterministic by
 * default and deterministic on request -- "aclnnGroupedMatmulFinalizeRouting
 * WeightNzV2", determinism notes for Atlas A2/A3). */
typedef enum {
  GMMFR_COMBINE_AUTO = 0,     /* library picks the fastest strategy            */
  GMMFR_COMBINE_ATOMIC = 1,   /* fp32 atomic adds from the GEMM epilogue       */
  GMMFR_COMBINE_ORDERED = 2,  /* rows sorted by destination, ordered reduction */
  GMMFR_COMBINE_HYBRID = 3    /* reported by the plan only (not a request):
                                 some 256-column tiles by atomics, the others
                                 by the ordered reduction, which then overlaps
                                 the atomics with the GEMM; order unspecified */
} gmmfr_combine;

/* Arguments.  Names follow the operator's parameter list. */
typedef struct {
  /* x1: INT8 (m,k), rows sorted by expert; FLOAT8_E4M3FN (m,k) selects the
   * MxA8W4 mode (Atlas 350 notes) when x2 is FP4, with the other inputs as
   * marked MX, or the FP8 mode when x2 is FLOAT8_E4M3FN (e,k,n), or (e,n,k)
   * with transpose_x2 = 1 (scale and pertokenScale as for INT8; rowIndex
   * INT64).                                                            required */
  gmmfr_tensor x1;
  /* x2: INT8 (e,k,n); or INT32 (e,k,n/8) holding eight int4 per word, column
   * 8w+t in bits [4t,4t+4); or INT4 (e,k,n), the same bytes.  With
   * transpose_x2 = 1: INT8 (e,n,k), weight column j of expert g at
   * x2[g][j][:] (parameter notes: (e,n,k) when transposed).
   * FP8: FLOAT8_E4M3FN (e,k,n), or (e,n,k) with transpose_x2 = 1.
   * MX: FLOAT4_E2M1X2 (e,n,k/2), i.e. (e,n,k) two per byte along k, with
   * transpose_x2 = 1.                                                  required */
  gmmfr_tensor x2;
  /* scale: FLOAT32 or BFLOAT16 (e,1,n) per-channel dequant scale.      optional
   * (INT64 scale is listed by the operator without an encoding: UNSUPPORTED)
   * MX: FLOAT8_E8M0 (e,n,k/64,2), the block scale of x2 for each 32 k of each
   * weight column.                                                     required */
  gmmfr_tensor scale;
  /* bias, offset, antiquantScale, antiquantOffset: reserved by the operator
   * ("pass a null pointer"); must be absent, else UNSUPPORTED.                 */
  gmmfr_tensor bias, offset, antiquant_scale, antiquant_offset;
  /* pertokenScale: FLOAT32 (m) per-token scale, or FLOAT32 (1): one static
   * per-tensor activation scale applied to every row (function description:
   * Atlas 350 static pertensor-perchannel quantisation).             optional
   * MX: FLOAT8_E8M0 (m,k/64,2), the block scale of x1 for each 32 k of each
   * row.                                                                required */
  gmmfr_tensor pertoken_scale;
  /* groupList: INT64 (e); type 0 cumulative ends, type 1 counts.       required */
  gmmfr_tensor group_list;
  /* sharedInput: BFLOAT16 (bsdp,n), bsdp <= outputBS.                  optional */
  gmmfr_tensor shared_input;
  /* logit: FLOAT32 (m) routing weight of each row.                     optional */
  gmmfr_tensor logit;
  /* rowIndex: INT64 or INT32 (m), destination row of each source row;
   * absent means the identity.  MX: INT64 only.                        optional */
  gmmfr_tensor row_index;
  /* out: FLOAT32 (outputBS,n); every element is written.               required */
  gmmfr_tensor out;
  /* acc_out: INT32 (m,n) copy of the int32 accumulators of covered rows
   * (other rows untouched).  A diagnostic for tests.  MX: UNSUPPORTED. optional */
  gmmfr_tensor acc_out;

  int64_t group_list_type;      /* 0 or 1                                        */
  int64_t shared_input_offset;  /* >= 0, offset + bsdp <= outputBS               */
  int64_t output_bs;            /* rows of out                                   */
  int32_t transpose_x1;         /* must be 0                                     */
  int32_t transpose_x2;         /* 0: x2 is (e,k,n); 1: INT8 x2 is (e,n,k) (int4
                                   weights transposed: UNSUPPORTED)              */
  int32_t deterministic;        /* 0: order of additions unspecified (default);
                                   1: bit-reproducible, rows folded in ascending
                                   source order onto the seed                    */
  int32_t combine;              /* gmmfr_combine; ATOMIC with deterministic=1 is
                                   rejected (ATTR)                               */
  /* tuningConfig: host array; element 0 = expected rows per expert, used only
   * to choose tiles ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", function
   * description: the first value is the expected token count per expert and
   * the tiling follows it).  Element 1 (an extension of this library), if
   * present and non-zero, forces the tile height: 32, 64, 128 or 256; any
   * other value is rejected (ATTR).  Element 2 (also ours, meant for tests),
   * if present and non-zero, caps the number of workgroups of the persistent
   * GEMM launch, so that each runs many tiles in a row; negative values are
   * rejected (ATTR).  Element 3 (ours, for tests) picks how the ordered
   * combine finds each destination's rows: 0 by problem size, 1 a bucket
   * index, 2 a scan of rowIndex per destination; other values are rejected
   * (ATTR).  Element 4 (ours, for tuning and tests), if present and
   * non-zero, asks for the hybrid combine with that many atomic column tiles
   * in every 8 consecutive 256-column tiles (1 .. 7; other values ATTR); it is
   * honoured only with combine AUTO, deterministic = 0, int8 or int4 weights
   * and a GEMM tile and k that run the continuous copy pipeline with it
   * (256 x 256 with k % 128 == 0, or 128 x 256), and ignored elsewhere.  AUTO
   * alone never takes the hybrid combine.  Results never depend on elements 0-4:
   * the int32 accumulators and the ordered combine are bit-identical for any
   * value, the unordered combines differ only in the order of their
   * additions.  May be NULL.                                                  */
  const int64_t* tuning_config;
  int64_t tuning_config_len;
} gmmfr_args;

/*
 * Limits of this implementation (beyond the operator's own rules):
 *   1 <= e <= 1024, 0 <= m < 2^31, 1 <= n, n % 16 == 0 (n % 32 == 0 for int4
 *   weights), 64 <= k <= 65536 with k % 64 == 0, outputBS >= 1,
 *   m * n < 2^40, every base pointer 16-byte aligned.
 * Device data are not validated (that would need a device-to-host read):
 *   a groupList that breaks its rule is clamped to [0, m] and made
 *   non-decreasing, rows whose rowIndex lies outside [0, outputBS) are
 *   skipped.  Such inputs give an unspecified result but no out-of-bounds
 *   access.
 */

/* Stage 1: validate `args` (host-side checks only, no device access, no HIP
 * call) and report the workspace size in bytes for stage 2.
 * Returns GMMFR_OK or the first rule broken. */
int gmm_finalize_routing_workspace(const gmmfr_args* args, size_t* workspace_bytes);

/* Stage 2: validate again, then enqueue the computation on `stream`
 * (a hipStream_t; NULL = the null stream).  `workspace` is device memory of
 * at least the stage-1 size: 1 KiB of work-queue counters in every mode, plus,
 * for the ordered combine, m*n*4 bytes of per-row contributions and
 * (2*outputBS + outputBS+1 + m) int32 of row buckets (256-byte aligned
 * sections).  Its contents need no initialisation and are not preserved.
 * Returns GMMFR_OK, a validation status, GMMFR_ERR_WORKSPACE, or
 * GMMFR_ERR_HIP when a launch fails. */
int gmm_finalize_routing(const gmmfr_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* Diagnostic variant of stage 2 for measurement: identical work, plus
 * hipEventRecord(gemm_start) right before and hipEventRecord(gemm_stop) right
 * after the grouped GEMM launch, on `stream`.  Both events are hipEvent_t
 * created by the caller (either may be NULL).  No event is recorded when the
 * call returns an error or when there is no GEMM launch (m == 0). */
int gmm_finalize_routing_profiled(const gmmfr_args* args, void* workspace, size_t workspace_bytes, void* stream,
                                  void* gemm_start, void* gemm_stop);

/* Allocation-free variant of stage 2, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Identical work and results to
 * gmm_finalize_routing, but the workspace is a device array inside the
 * library, GMMFR_NOALLOC_SCRATCH_BYTES long, which each GPU the library runs
 * on holds from its first use until the process ends; the call itself
 * allocates and frees nothing.  The caller still passes every input and
 * output.  A plan that needs more workspace than the array holds is rejected
 * with GMMFR_ERR_WORKSPACE before any device work (the ordered combine needs
 * about m*n*4 bytes: force combine = GMMFR_COMBINE_ATOMIC, whose plan needs
 * 1 KiB, or use gmm_finalize_routing).  Every call on one GPU shares that
 * GPU's array and the kernels re-initialise what they use, so calls that
 * overlap on one GPU (on different streams, or from different host threads
 * without ordering) race and give wrong results; calls ordered on one stream
 * are safe.  Returns as gmm_finalize_routing; GMMFR_ERR_HIP also when the
 * array's device address cannot be obtained. */
#define GMMFR_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int gmm_finalize_routing_noalloc(const gmmfr_args* args, void* stream);

/* Description of the plan stage 2 would use for `args` (host only). */
typedef struct {
  int32_t combine;          /* gmmfr_combine actually used (ATOMIC, ORDERED or
                               HYBRID)                                         */
  int32_t tile_m, tile_n;   /* GEMM block tile                                 */
  int32_t tile_k;           /* k step per pipeline stage                       */
  int32_t grid;             /* workgroups of the grouped GEMM launch           */
  int32_t int4_weights;     /* 1 if x2 is int4                                 */
  int64_t workspace_bytes;
  char gemm_kernel[96];     /* symbol-like name of the GEMM kernel variant     */
  int32_t hybrid_atomic;    /* HYBRID: atomic column tiles in every 8, else 0  */
} gmmfr_plan_info;

int gmm_finalize_routing_plan(const gmmfr_args* args, gmmfr_plan_info* info);

/*
 * Producer step: dynamic per-token int8 quantisation of bf16 hidden states and
 * the routing permute, which together make this library's x1, pertokenScale,
 * logit, rowIndex and groupList from a router's top-K choice.  The pages name
 * the step ("aclnnAlltoAllvQuantGroupedMatMul", function and formula: a
 * permute after the dispatch, before the expert matmul; quantisation modes:
 * per-token dynamic quantisation) and show the per-token cast multiplying by
 * an inverse scale (PTOAS issue #1568, background); the formulas are lost, so
 * the plain symmetric reading is taken:
 *
 *   per token t (x = its k bf16 values widened to fp32):
 *     amax = max_j |x[j]|,  scale_t = fl(amax / 127),  inv = fl(127 / amax)
 *     (inv = 0 when amax = 0),  q[j] = clamp(rne(fl(x[j] * inv)), -127, 127)
 *   entry f = t*K + j goes to local expert g = expert_ids[t][j] - expert_offset;
 *   entries with g outside [0, e) produce no row (they belong to other ranks);
 *   rows are the local entries sorted by g, ties in ascending f; the row of
 *   entry f gets x1 = q of token t, pertokenScale = scale_t,
 *   logit = topk_weights[t][j], rowIndex = t;
 *   groupList[g] = rows of expert g (type 1) or their cumulative end (type 0).
 *
 * FP8 x1 (readings; 448 is the largest E4M3 value, E4M3(v) rounds to nearest,
 * ties to even):
 *   with FLOAT32 pertokenScale: scale_t = fl(amax / 448), codes of
 *     E4M3(clamp(fl(x * fl(448 / amax)), -448, 448));
 *   with FLOAT8_E8M0 pertokenScale (the OCP MX conversion, per 32 values of a
 *     token): shared exponent s = floor(log2(block amax)) - 8, clamped to
 *     [-127, 127] (-127 for an all-zero block), E8M0 code s + 127, codes of
 *     E4M3(clamp(x * 2^-s, -448, 448)).
 *
 * Rows at and past sum(groupList counts) are not written (the grouped matmul
 * never reads them).  Hidden values must be finite; expert ids are device data
 * and are not validated beyond routing the out-of-range ones nowhere.
 */
typedef struct {
  gmmfr_tensor hidden;         /* BFLOAT16 (T,k)                                required */
  gmmfr_tensor expert_ids;     /* INT32 or INT64 (T,K): global expert per slot  required */
  gmmfr_tensor topk_weights;   /* FLOAT32 (T,K) routing weights; given iff logit is given */
  gmmfr_tensor x1;             /* out INT8 (T*K,k), or FLOAT8_E4M3FN (T*K,k)    required */
  gmmfr_tensor pertoken_scale; /* out FLOAT32 (T*K); with FP8 x1 FLOAT32 (T*K), or
                                * FLOAT8_E8M0 (T*K, k/64, 2): one scale per 32
                                * values (MX; k % 64 == 0)                     required */
  gmmfr_tensor logit;          /* out FLOAT32 (T*K); given iff topk_weights is given      */
  gmmfr_tensor row_index;      /* out INT64 or INT32 (T*K)                      required */
  gmmfr_tensor group_list;     /* out INT64 (e)                                 required */
  int64_t expert_offset;       /* local experts are [expert_offset, expert_offset + e)    */
  int64_t group_list_type;     /* 0 cumulative ends, 1 counts                             */
} gmmqp_args;

/* Limits: 0 <= T, 1 <= K <= 64, T*K < 2^31, 16 <= k <= 65536 with k % 16 == 0,
 * 1 <= e <= 1024, every base pointer 16-byte aligned.
 * Stage 1: validate (host only) and report the workspace size: one int32 per
 * (expert, chunk of 256 entries), one per expert and T*K more, in 256-byte
 * aligned sections. */
int gmm_quant_permute_workspace(const gmmqp_args* args, size_t* workspace_bytes);

/* Stage 2: validate again and enqueue on `stream` (hipStream_t; NULL = null
 * stream).  Every output is caller-owned device memory; the workspace needs no
 * initialisation.  Returns GMMFR_OK, a validation status, GMMFR_ERR_WORKSPACE
 * or GMMFR_ERR_HIP. */
int gmm_quant_permute(const gmmqp_args* args, void* workspace, size_t workspace_bytes, void* stream);

/* Diagnostic variant of gmm_quant_permute for measurement: identical work,
 * plus hipEventRecord(quant_start) right before and hipEventRecord(quant_stop)
 * right after the quantisation kernel, on `stream` (caller-created hipEvent_t,
 * either may be NULL; none recorded on error or when T == 0). */
int gmm_quant_permute_profiled(const gmmqp_args* args, void* workspace, size_t workspace_bytes, void* stream,
                               void* quant_start, void* quant_stop);

/* Short static text for a status code. */
const char* gmmfr_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* GMMFR_H */
