/*
 * Reference oracle: plain, slow, obviously correct CPU evaluation of the
 * fused quantized MoE grouped matmul + finalize-routing combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the GPU path includes, links or calls
 * this file; the two share no code.  Built with
 *     gcc -O3 -fno-fast-math -ffp-contract=off -fopenmp
 * so every float operation is one IEEE-754 binary32 operation rounded to
 * nearest-even, in the order written (no FMA contraction, no reassociation).
 *
 * The steps below follow the reading stated in gmmfr_oracle.h, in this order:
 *   1 validate   2 expand groupList   3 int32 GEMM per group
 *   4 dequantise 5 seed the output    6 combine by rowIndex (ascending row)
 */
#include "gmmfr_oracle.h"

#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- helpers */

/* bf16 -> fp32 widening is exact: the 16 stored bits are the high half of
 * the fp32 pattern. */
static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Destination row of source row i: rowIndex[i], or i when rowIndex is absent
 * (aclnnGroupedMatmulFinalizeRoutingWeightNzV2, parameter notes: rowIndex is
 * optional on Atlas A2/A3 and INT64 or INT32). */
static int64_t dest_of(const orc_problem* p, int64_t i) {
  if (!p->row_index) return i;
  if (p->row_index_type == ORC_I64) return ((const int64_t*)p->row_index)[i];
  return (int64_t)((const int32_t*)p->row_index)[i];
}

/* Weight W_g[kk][j] as a signed integer.  int8 x2 is (e,k,n) row-major.  For
 * the packed form (e,k,n/8) int32, column j is nibble (j mod 8) of word
 * floor(j/8), low nibble first, two's complement in [-8, 7]. */
static int32_t weight_at(const orc_problem* p, int64_t g, int64_t kk, int64_t j) {
  if (p->x2_type == ORC_I8) {
    const int8_t* w = (const int8_t*)p->x2;
    return (int32_t)w[(g * p->k + kk) * p->n + j];
  }
  const uint32_t* w = (const uint32_t*)p->x2;
  uint32_t word = w[(g * p->k + kk) * (p->n / 8) + j / 8];
  int32_t nib = (int32_t)((word >> (4 * (j % 8))) & 0xFu);
  return nib >= 8 ? nib - 16 : nib;
}

/* Per-channel scale S_g[j] widened to fp32; absent => 1. */
static float scale_at(const orc_problem* p, int64_t g, int64_t j) {
  if (!p->scale) return 1.0f;
  if (p->scale_type == ORC_F32) return ((const float*)p->scale)[g * p->n + j];
  return bf16_to_f32(((const uint16_t*)p->scale)[g * p->n + j]);
}

/* Step 4: y = ((float(acc) * S_g[j]) * P_i) * L_i, each product rounded to
 * fp32.  The (acc * deqScale) * perTokenScale order is the one the worked
 * example of "matmul支持pertoken量化模式" spells out; the routing weight
 * (logit) comes last.  A missing factor is 1.0, and x * 1.0f == x exactly.
 * A per-tensor pertokenScale ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2",
 * function description: static pertensor-perchannel) is P_i = P_0 for all i. */
static float dequant(const orc_problem* p, int64_t g, int64_t i, int64_t j, int32_t acc) {
  float y = (float)acc;             /* int32 -> fp32, round to nearest even */
  y = y * scale_at(p, g, j);
  y = y * (p->pertoken_scale ? p->pertoken_scale[p->pertoken_per_tensor ? 0 : i] : 1.0f);
  y = y * (p->logit ? p->logit[i] : 1.0f);
  return y;
}

/* Step 5 value for element (d, j): +0.0f, or the widened sharedInput block
 * placed at rows [offset, offset + bsdp).  ("aclnnGroupedMatmulFinalizeRouting
 * WeightNzV2", Atlas 350 common constraints: bsdp <= outputBS and
 * sharedInputOffset + bsdp <= outputBS.) */
static float seed_at(const orc_problem* p, int64_t d, int64_t j) {
  if (p->shared_input && d >= p->shared_input_offset && d < p->shared_input_offset + p->bsdp)
    return bf16_to_f32(p->shared_input[(d - p->shared_input_offset) * p->n + j]);
  return 0.0f;
}

/* Step 2: group ranges.  ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2",
 * common constraints: type 0 is a non-negative non-decreasing list of
 * cumulative ends; type 1 is a list of non-negative per-expert counts.) */
int orc_group_ranges(const orc_problem* p, int64_t* start, int64_t* end) {
  int64_t prev = 0;
  for (int64_t g = 0; g < p->e; ++g) {
    int64_t v = p->group_list[g];
    if (v < 0) return ORC_ERR_GROUPLIST;
    if (p->group_list_type == 0) {
      if (v < prev) return ORC_ERR_GROUPLIST;
      start[g] = prev;
      end[g] = v;
    } else {
      start[g] = prev;
      end[g] = prev + v;
    }
    if (end[g] > p->m) return ORC_ERR_GROUPLIST;  /* more rows than x1 holds */
    prev = end[g];
  }
  return ORC_OK;
}

/* Step 1: strict validation of arguments and of the data contract. */
static int validate(const orc_problem* p, int64_t* start, int64_t* end) {
  if (!p || !p->x1 || !p->x2 || !p->group_list) return ORC_ERR_NULL;
  if (p->m < 0 || p->k < 1 || p->n < 1 || p->e < 1 || p->output_bs < 0) return ORC_ERR_SHAPE;
  if (p->x2_type != ORC_I8 && p->x2_type != ORC_I4PACKED) return ORC_ERR_DTYPE;
  if (p->x2_type == ORC_I4PACKED && p->n % 8 != 0) return ORC_ERR_SHAPE;
  if (p->scale && p->scale_type != ORC_F32 && p->scale_type != ORC_BF16) return ORC_ERR_DTYPE;
  if (p->row_index && p->row_index_type != ORC_I64 && p->row_index_type != ORC_I32) return ORC_ERR_DTYPE;
  if (p->group_list_type != 0 && p->group_list_type != 1) return ORC_ERR_GROUPLIST;
  if (p->shared_input) {
    if (p->bsdp < 0 || p->shared_input_offset < 0 || p->bsdp > p->output_bs ||
        p->shared_input_offset + p->bsdp > p->output_bs)
      return ORC_ERR_SHARED;
  }
  int st = orc_group_ranges(p, start, end);
  if (st != ORC_OK) return st;
  for (int64_t g = 0; g < p->e; ++g)
    for (int64_t i = start[g]; i < end[g]; ++i) {
      int64_t d = dest_of(p, i);
      if (d < 0 || d >= p->output_bs) return ORC_ERR_ROWINDEX;
    }
  return ORC_OK;
}

/* Step 3 for one row: acc[j] = sum_kk int32(x1[i][kk]) * int32(W_g[kk][j]).
 * |acc| <= k * 128 * 128, exact in int32 for k <= 2^17. */
static void acc_row(const orc_problem* p, int64_t g, int64_t i, int32_t* acc, int32_t* wrow) {
  for (int64_t j = 0; j < p->n; ++j) acc[j] = 0;
  for (int64_t kk = 0; kk < p->k; ++kk) {
    int32_t a = (int32_t)p->x1[i * p->k + kk];
    for (int64_t j = 0; j < p->n; ++j) wrow[j] = weight_at(p, g, kk, j);
    for (int64_t j = 0; j < p->n; ++j) acc[j] += a * wrow[j];
  }
}

/* ------------------------------------------------------------ entry points */

int orc_gmm_finalize_routing(const orc_problem* p, float* out, int32_t* acc_dump) {
  if (!out) return ORC_ERR_NULL;
  int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(p ? (p->e > 0 ? p->e : 1) : 1));
  int64_t* end = (int64_t*)malloc(sizeof(int64_t) * (size_t)(p ? (p->e > 0 ? p->e : 1) : 1));
  int st = validate(p, start, end);
  if (st != ORC_OK) { free(start); free(end); return st; }
  const int64_t m = p->m, n = p->n, e = p->e;

  /* expert of each row; -1 for rows outside every group */
  int64_t* group_of = (int64_t*)malloc(sizeof(int64_t) * (size_t)(m > 0 ? m : 1));
  for (int64_t i = 0; i < m; ++i) group_of[i] = -1;
  for (int64_t g = 0; g < e; ++g)
    for (int64_t i = start[g]; i < end[g]; ++i) group_of[i] = g;

  /* Step 3: int32 accumulators (uncovered rows stay 0) */
  int32_t* acc = acc_dump ? acc_dump : (int32_t*)malloc(sizeof(int32_t) * (size_t)(m * n > 0 ? m * n : 1));
#pragma omp parallel
  {
    int32_t* wrow = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
#pragma omp for schedule(dynamic, 4)
    for (int64_t i = 0; i < m; ++i) {
      if (group_of[i] < 0) {
        for (int64_t j = 0; j < n; ++j) acc[i * n + j] = 0;
      } else {
        acc_row(p, group_of[i], i, acc + i * n, wrow);
      }
    }
    free(wrow);
  }

  /* Step 4: dequantised contributions of covered rows */
  float* y = (float*)malloc(sizeof(float) * (size_t)(m * n > 0 ? m * n : 1));
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < m; ++i)
    if (group_of[i] >= 0)
      for (int64_t j = 0; j < n; ++j) y[i * n + j] = dequant(p, group_of[i], i, j, acc[i * n + j]);

  /* Step 5: seed */
#pragma omp parallel for schedule(static)
  for (int64_t d = 0; d < p->output_bs; ++d)
    for (int64_t j = 0; j < n; ++j) out[d * n + j] = seed_at(p, d, j);

  /* Step 6: combine.  Each element is a left fold over its source rows in
   * ascending row order; threads split the columns, never the rows, so the
   * order per element is exactly that fold. */
  const int64_t JB = 256;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t jb = 0; jb < n; jb += JB) {
    int64_t je = jb + JB < n ? jb + JB : n;
    for (int64_t i = 0; i < m; ++i) {
      if (group_of[i] < 0) continue;
      int64_t d = dest_of(p, i);
      for (int64_t j = jb; j < je; ++j) out[d * n + j] = out[d * n + j] + y[i * n + j];
    }
  }

  free(y);
  if (!acc_dump) free(acc);
  free(group_of);
  free(start);
  free(end);
  return ORC_OK;
}

int orc_out_rows(const orc_problem* p, int64_t count, const int64_t* d_list, float* out_rows) {
  if (!out_rows || (count > 0 && !d_list)) return ORC_ERR_NULL;
  int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(p ? (p->e > 0 ? p->e : 1) : 1));
  int64_t* end = (int64_t*)malloc(sizeof(int64_t) * (size_t)(p ? (p->e > 0 ? p->e : 1) : 1));
  int st = validate(p, start, end);
  if (st != ORC_OK) { free(start); free(end); return st; }
  for (int64_t c = 0; c < count; ++c)
    if (d_list[c] < 0 || d_list[c] >= p->output_bs) { free(start); free(end); return ORC_ERR_ROWINDEX; }
  const int64_t n = p->n;
#pragma omp parallel
  {
    int32_t* acc = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    int32_t* wrow = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
#pragma omp for schedule(dynamic, 1)
    for (int64_t c = 0; c < count; ++c) {
      const int64_t d = d_list[c];
      float* o = out_rows + c * n;
      for (int64_t j = 0; j < n; ++j) o[j] = seed_at(p, d, j);
      /* covered source rows with destination d, ascending */
      for (int64_t g = 0; g < p->e; ++g)
        for (int64_t i = start[g]; i < end[g]; ++i) {
          if (dest_of(p, i) != d) continue;
          acc_row(p, g, i, acc, wrow);
          for (int64_t j = 0; j < n; ++j) o[j] = o[j] + dequant(p, g, i, j, acc[j]);
        }
    }
    free(acc);
    free(wrow);
  }
  free(start);
  free(end);
  return ORC_OK;
}

int orc_acc_rows(const orc_problem* p, int64_t count, const int64_t* i_list, int32_t* acc_rows) {
  if (!acc_rows || (count > 0 && !i_list)) return ORC_ERR_NULL;
  int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(p ? (p->e > 0 ? p->e : 1) : 1));
  int64_t* end = (int64_t*)malloc(sizeof(int64_t) * (size_t)(p ? (p->e > 0 ? p->e : 1) : 1));
  int st = validate(p, start, end);
  if (st != ORC_OK) { free(start); free(end); return st; }
  for (int64_t c = 0; c < count; ++c)
    if (i_list[c] < 0 || i_list[c] >= p->m) { free(start); free(end); return ORC_ERR_SHAPE; }
  const int64_t n = p->n;
#pragma omp parallel
  {
    int32_t* wrow = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
#pragma omp for schedule(dynamic, 1)
    for (int64_t c = 0; c < count; ++c) {
      const int64_t i = i_list[c];
      int64_t g = -1;
      for (int64_t h = 0; h < p->e; ++h)
        if (i >= start[h] && i < end[h]) g = h;
      if (g < 0) {
        for (int64_t j = 0; j < n; ++j) acc_rows[c * n + j] = 0;
      } else {
        acc_row(p, g, i, acc_rows + c * n, wrow);
      }
    }
    free(wrow);
  }
  free(start);
  free(end);
  return ORC_OK;
}
