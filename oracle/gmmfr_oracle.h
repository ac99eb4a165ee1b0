/*
 * Reference oracle for the fused quantized MoE grouped matmul with
 * finalize-routing combine.  TEST INFRASTRUCTURE ONLY: tests, the smoke check
 * and the CPU-baseline leg of the benchmark may call it; the GPU library never
 * does, and the two share no code.
 *
 * What it computes (sources are the pages' titles and sections):
 *   - "aclnnGroupedMatmulFinalizeRoutingWeightNzV2" (CANN operator doc),
 *     function description: a GroupedMatmul whose output is combined by index
 *     (MoeFinalizeRouting); parameter notes (Atlas A2/A3) give x1 int8 (m,k),
 *     x2 int8 (e,k,n) or int4 packed eight-per-int32 as (e,k,n/8), scale
 *     FLOAT/BF16 (e,1,n), rowIndex INT64/INT32; constraints give the groupList
 *     rule (type 0 cumulative non-decreasing, type 1 non-negative counts) and,
 *     for sharedInput, bsdp <= outputBS and offset + bsdp <= outputBS.
 *   - "matmul支持pertoken量化模式" (ATB per-token quantised linear), worked
 *     example: out[i][j] = (sum_k x[i][k] * w[k][j]) * deqScale[j] *
 *     perTokenScale[i], applied left to right.
 *
 * Readings taken where the pages are silent (each listed with its reason in
 * the design notes of the repository):
 *   - epilogue in IEEE fp32, each product rounded:  y = ((float(acc) * S) * P) * L,
 *     with float() the round-to-nearest-even int32 -> fp32 conversion and an
 *     absent factor equal to 1;
 *   - the output starts at +0.0f, rows [off, off+bsdp) seeded with the
 *     widened bf16 sharedInput; every covered source row i is then added into
 *     out[rowIndex[i]] in ascending i (the deterministic order);
 *   - rows after the last group end contribute nothing; absent rowIndex is the
 *     identity; int4 nibble t of a packed word is column 8w+t, low nibble
 *     first, two's complement.
 */
#ifndef GMMFR_ORACLE_H
#define GMMFR_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types (independent numbering from the GPU library's) */
enum { ORC_NONE = 0, ORC_I8 = 1, ORC_I32 = 2, ORC_I64 = 3, ORC_F32 = 4, ORC_BF16 = 5, ORC_I4PACKED = 6 };

/* status codes: 0 ok, otherwise the first violated rule */
enum {
  ORC_OK = 0,
  ORC_ERR_NULL = 1,        /* required array missing                      */
  ORC_ERR_DTYPE = 2,       /* unsupported element type                    */
  ORC_ERR_SHAPE = 3,       /* sizes inconsistent                          */
  ORC_ERR_GROUPLIST = 4,   /* groupList breaks its rule or exceeds m      */
  ORC_ERR_ROWINDEX = 5,    /* rowIndex outside [0, outputBS)              */
  ORC_ERR_SHARED = 6,      /* sharedInput block outside the output        */
};

typedef struct {
  int64_t m, k, n, e;
  const int8_t* x1;            /* (m,k) row-major                                   */
  const void* x2;              /* ORC_I8: (e,k,n) int8 ; ORC_I4PACKED: (e,k,n/8) i32 */
  int32_t x2_type;
  const void* scale;           /* (e,1,n) ORC_F32 or ORC_BF16 (raw bits) ; or NULL */
  int32_t scale_type;
  const float* pertoken_scale; /* (m) or NULL                                      */
  const float* logit;          /* (m) or NULL                                      */
  const int64_t* group_list;   /* (e)                                              */
  int64_t group_list_type;     /* 0 cumulative, 1 counts                           */
  const void* row_index;       /* (m) ORC_I64 or ORC_I32 ; or NULL (identity)      */
  int32_t row_index_type;
  const uint16_t* shared_input;/* (bsdp,n) bf16 raw bits ; or NULL                 */
  int64_t bsdp;
  int64_t shared_input_offset;
  int64_t output_bs;
  int32_t pertoken_per_tensor; /* 1: pertoken_scale holds one value, used for every
                                * row (static per-tensor activation scale)     */
} orc_problem;

/* Whole computation: out (output_bs,n) fp32, fully written; acc (m,n) int32
 * dump (rows outside every group are 0), may be NULL. */
int orc_gmm_finalize_routing(const orc_problem* p, float* out, int32_t* acc);

/* Same definition evaluated only for the listed destination rows d_list[c]
 * (out_rows is count x n).  Used to check full-size runs on samples. */
int orc_out_rows(const orc_problem* p, int64_t count, const int64_t* d_list, float* out_rows);

/* int32 accumulator of the listed source rows (acc_rows is count x n). */
int orc_acc_rows(const orc_problem* p, int64_t count, const int64_t* i_list, int32_t* acc_rows);

/* Group ranges [start_g, end_g) from groupList; returns status. */
int orc_group_ranges(const orc_problem* p, int64_t* start, int64_t* end);

#ifdef __cplusplus
}
#endif
#endif
