// C-ABI entry points: argument validation, planning, launch.
//
// Two-stage use as in "aclnnGroupedMatmulFinalizeRoutingWeightNzV2"
// (interface description): the first call validates the arguments and sizes
// the workspace, the second enqueues the work on a stream.  No executor object
// is kept: the second call re-derives the same plan from the same arguments.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/gmmfr.h"
#include "gmmfr_internal.h"

namespace {

using namespace gmmfr;

struct Derived {
  int64_t m, k, n, e, bsdp, output_bs;
  bool int4;
  bool trans_b;  // int8 weights given transposed, (e,n,k)
  bool mx;       // MxA8W4: FP8 x1, FP4 x2 (e,n,k), E8M0 block scales
  bool fp8;      // FP8 x1 and x2 (e,n,k), per-channel scale, per-token pertokenScale
  bool scale_bf16;
  bool pts_scalar;  // pertokenScale of shape (1): one static per-tensor activation scale
  bool row_index_i32;
};

// A tensor is given when it has data, or when it has no elements at all (an
// allocator may hand out a null pointer for zero bytes).
bool present(const gmmfr_tensor& t) {
  if (t.data != nullptr) return true;
  for (int i = 0; i < t.ndim && i < 4; ++i)
    if (t.dims[i] == 0) return true;
  return false;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool dims_are(const gmmfr_tensor& t, int nd, int64_t d0, int64_t d1 = -1, int64_t d2 = -1, int64_t d3 = -1) {
  if (t.ndim != nd) return false;
  const int64_t want[4] = {d0, d1, d2, d3};
  for (int i = 0; i < nd; ++i)
    if (t.dims[i] != want[i]) return false;
  return true;
}

// Attribute rules common to both data paths.
int check_attributes(const gmmfr_args* a) {
  if (a->group_list_type != 0 && a->group_list_type != 1) return GMMFR_ERR_ATTR;
  if (a->deterministic != 0 && a->deterministic != 1) return GMMFR_ERR_ATTR;
  if (a->combine != GMMFR_COMBINE_AUTO && a->combine != GMMFR_COMBINE_ATOMIC && a->combine != GMMFR_COMBINE_ORDERED)
    return GMMFR_ERR_ATTR;
  if (a->deterministic == 1 && a->combine == GMMFR_COMBINE_ATOMIC) return GMMFR_ERR_ATTR;
  if (a->tuning_config_len < 0 || (a->tuning_config_len > 0 && !a->tuning_config)) return GMMFR_ERR_ATTR;
  if (a->tuning_config_len > 1 && a->tuning_config[1] != 0 && a->tuning_config[1] != 32 &&
      a->tuning_config[1] != 64 && a->tuning_config[1] != 128 && a->tuning_config[1] != 256)
    return GMMFR_ERR_ATTR;
  // element 2: cap on the persistent GEMM's workgroups (0 = none)
  if (a->tuning_config_len > 2 && (a->tuning_config[2] < 0 || a->tuning_config[2] >= (int64_t(1) << 31)))
    return GMMFR_ERR_ATTR;
  // element 3: the ordered combine's row lookup (0 = by size, 1 = bucket index, 2 = scan)
  if (a->tuning_config_len > 3 && (a->tuning_config[3] < 0 || a->tuning_config[3] > 2)) return GMMFR_ERR_ATTR;
  // element 4: hybrid combine with that many atomic column tiles in each kHybridPeriod (0 = AUTO's choice)
  if (a->tuning_config_len > 4 && (a->tuning_config[4] < 0 || a->tuning_config[4] >= kHybridPeriod))
    return GMMFR_ERR_ATTR;
  return GMMFR_OK;
}

// out (outputBS,n), sharedInput placement and the alignment of every present
// base pointer, common to both data paths.
int check_output_and_alignment(const gmmfr_args* a, int64_t n, int64_t* bsdp) {
  const int64_t obs = a->output_bs;
  if (obs < 1 || obs >= (int64_t(1) << 31)) return GMMFR_ERR_SHAPE;
  if (!dims_are(a->out, 2, obs, n)) return GMMFR_ERR_SHAPE;
  *bsdp = 0;
  if (present(a->shared_input)) {
    if (a->shared_input.ndim != 2 || a->shared_input.dims[1] != n) return GMMFR_ERR_SHAPE;
    *bsdp = a->shared_input.dims[0];
    // bsdp <= outputBS and sharedInputOffset + bsdp <= outputBS (Atlas 350 common constraints)
    if (*bsdp < 0 || *bsdp > obs) return GMMFR_ERR_ATTR;
    if (a->shared_input_offset < 0 || a->shared_input_offset + *bsdp > obs) return GMMFR_ERR_ATTR;
  } else if (a->shared_input_offset < 0) {
    return GMMFR_ERR_ATTR;
  }
  const gmmfr_tensor* all[] = {&a->x1, &a->x2, &a->scale, &a->pertoken_scale, &a->group_list, &a->shared_input,
                               &a->logit, &a->row_index, &a->out, &a->acc_out};
  for (const gmmfr_tensor* t : all)
    if (present(*t) && !aligned16(t->data)) return GMMFR_ERR_ALIGN;
  return GMMFR_OK;
}

// MxA8W4 ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", Atlas 350 notes on
// the MxA8W4 quantisation: x2 (e,n,k) with transposeX2 fixed true,
// pertokenScale required with shape (m, ceil(k/64), 2), scale shape
// (e, n, ceil(k/64), 2), k % 32 == 0, n % 32 == 0; rowIndex INT64 only).
// Reading of the lost dtype table: x1 FLOAT8_E4M3FN, x2 FLOAT4_E2M1 two per
// byte along k, both scales FLOAT8_E8M0 (one per 32 k; when k % 64 == 32 the
// second byte of each row's last pair stands for no block and is ignored).
int validate_mx(const gmmfr_args* a, Derived* d) {
  if (!present(a->pertoken_scale) || !present(a->scale)) return GMMFR_ERR_NULLPTR;
  if (a->x2.dtype != GMMFR_DT_FLOAT4_E2M1X2) return GMMFR_ERR_DTYPE;
  if (a->pertoken_scale.dtype != GMMFR_DT_FLOAT8_E8M0 || a->scale.dtype != GMMFR_DT_FLOAT8_E8M0)
    return GMMFR_ERR_DTYPE;
  if (a->group_list.dtype != GMMFR_DT_INT64) return GMMFR_ERR_DTYPE;
  if (present(a->shared_input) && a->shared_input.dtype != GMMFR_DT_BFLOAT16) return GMMFR_ERR_DTYPE;
  if (present(a->logit) && a->logit.dtype != GMMFR_DT_FLOAT32) return GMMFR_ERR_DTYPE;
  if (present(a->row_index) && a->row_index.dtype != GMMFR_DT_INT64) return GMMFR_ERR_DTYPE;
  if (a->out.dtype != GMMFR_DT_FLOAT32) return GMMFR_ERR_DTYPE;
  if (present(a->acc_out)) return GMMFR_ERR_UNSUPPORTED;  // no integer accumulator on this path

  if (const int st = check_attributes(a)) return st;
  if (a->transpose_x1 != 0 || a->transpose_x2 != 1) return GMMFR_ERR_ATTR;

  if (a->x1.ndim != 2 || a->x2.ndim != 3) return GMMFR_ERR_SHAPE;
  const int64_t m = a->x1.dims[0], k = a->x1.dims[1];
  const int64_t e = a->x2.dims[0], n = a->x2.dims[1];
  if (a->x2.dims[2] * 2 != k) return GMMFR_ERR_SHAPE;
  if (m < 0 || m >= (int64_t(1) << 31)) return GMMFR_ERR_SHAPE;
  if (e < 1 || e > kMaxExperts) return GMMFR_ERR_SHAPE;
  if (k < 32 || k > 65536 || k % 32 != 0) return GMMFR_ERR_SHAPE;
  if (n < 32 || n % 32 != 0) return GMMFR_ERR_SHAPE;
  if (n > (int64_t(1) << 24) || m * n >= (int64_t(1) << 40)) return GMMFR_ERR_SHAPE;
  if (!dims_are(a->pertoken_scale, 3, m, (k + 63) / 64, 2)) return GMMFR_ERR_SHAPE;
  if (!dims_are(a->scale, 4, e, n, (k + 63) / 64, 2)) return GMMFR_ERR_SHAPE;
  if (!dims_are(a->group_list, 1, e)) return GMMFR_ERR_SHAPE;
  if (present(a->logit) && !dims_are(a->logit, 1, m)) return GMMFR_ERR_SHAPE;
  if (present(a->row_index) && !dims_are(a->row_index, 1, m)) return GMMFR_ERR_SHAPE;
  int64_t bsdp = 0;
  if (const int st = check_output_and_alignment(a, n, &bsdp)) return st;
  if (d) {
    d->m = m;
    d->k = k;
    d->n = n;
    d->e = e;
    d->bsdp = bsdp;
    d->output_bs = a->output_bs;
    d->int4 = false;
    d->trans_b = true;
    d->mx = true;
    d->fp8 = false;
    d->scale_bf16 = false;
    d->pts_scalar = false;
    d->row_index_i32 = false;
  }
  return GMMFR_OK;
}

// FP8 E4M3 x1 and x2 ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", parameter
// notes: rowIndex INT64 only when x1 and x2 are FLOAT8_E4M3FN; Atlas 350
// pertoken-perchannel quantisation): scale FLOAT32/BFLOAT16 (e,1,n) and
// pertokenScale FLOAT32 (m) as in the int8 mode; x2 (e,k,n), or (e,n,k) with
// transpose_x2 = 1 (full-quant notes).  Ours: k % 64 == 0, n % 16 == 0.
int validate_fp8(const gmmfr_args* a, Derived* d) {
  if (a->x2.dtype != GMMFR_DT_FLOAT8_E4M3FN) return GMMFR_ERR_DTYPE;
  if (present(a->scale) && a->scale.dtype != GMMFR_DT_FLOAT32 && a->scale.dtype != GMMFR_DT_BFLOAT16)
    return GMMFR_ERR_DTYPE;
  if (present(a->pertoken_scale) && a->pertoken_scale.dtype != GMMFR_DT_FLOAT32) return GMMFR_ERR_DTYPE;
  if (a->group_list.dtype != GMMFR_DT_INT64) return GMMFR_ERR_DTYPE;
  if (present(a->shared_input) && a->shared_input.dtype != GMMFR_DT_BFLOAT16) return GMMFR_ERR_DTYPE;
  if (present(a->logit) && a->logit.dtype != GMMFR_DT_FLOAT32) return GMMFR_ERR_DTYPE;
  if (present(a->row_index) && a->row_index.dtype != GMMFR_DT_INT64) return GMMFR_ERR_DTYPE;
  if (a->out.dtype != GMMFR_DT_FLOAT32) return GMMFR_ERR_DTYPE;
  if (present(a->acc_out)) return GMMFR_ERR_UNSUPPORTED;  // no integer accumulator on this path

  if (const int st = check_attributes(a)) return st;
  if (a->transpose_x1 != 0) return GMMFR_ERR_ATTR;
  // x2 (e,k,n), or (e,n,k) when transposed (full-quant notes)
  if (a->transpose_x2 != 0 && a->transpose_x2 != 1) return GMMFR_ERR_ATTR;
  const bool trans_b = a->transpose_x2 == 1;

  if (a->x1.ndim != 2 || a->x2.ndim != 3) return GMMFR_ERR_SHAPE;
  const int64_t m = a->x1.dims[0], k = a->x1.dims[1];
  const int64_t e = a->x2.dims[0], n = a->x2.dims[trans_b ? 1 : 2];
  if (a->x2.dims[trans_b ? 2 : 1] != k) return GMMFR_ERR_SHAPE;
  if (m < 0 || m >= (int64_t(1) << 31)) return GMMFR_ERR_SHAPE;
  if (e < 1 || e > kMaxExperts) return GMMFR_ERR_SHAPE;
  if (k < 64 || k > 65536 || k % 64 != 0) return GMMFR_ERR_SHAPE;
  if (n < 16 || n % 16 != 0) return GMMFR_ERR_SHAPE;
  if (n > (int64_t(1) << 24) || m * n >= (int64_t(1) << 40)) return GMMFR_ERR_SHAPE;
  if (present(a->scale) && !dims_are(a->scale, 3, e, 1, n)) return GMMFR_ERR_SHAPE;
  // pertokenScale (m) per token, or (1): the static per-tensor activation
  // scale (function description: Atlas 350 static pertensor-perchannel)
  if (present(a->pertoken_scale) && !dims_are(a->pertoken_scale, 1, m) && !dims_are(a->pertoken_scale, 1, 1))
    return GMMFR_ERR_SHAPE;
  if (!dims_are(a->group_list, 1, e)) return GMMFR_ERR_SHAPE;
  if (present(a->logit) && !dims_are(a->logit, 1, m)) return GMMFR_ERR_SHAPE;
  if (present(a->row_index) && !dims_are(a->row_index, 1, m)) return GMMFR_ERR_SHAPE;
  int64_t bsdp = 0;
  if (const int st = check_output_and_alignment(a, n, &bsdp)) return st;
  if (d) {
    d->m = m;
    d->k = k;
    d->n = n;
    d->e = e;
    d->bsdp = bsdp;
    d->output_bs = a->output_bs;
    d->int4 = false;
    d->trans_b = trans_b;
    d->mx = false;
    d->fp8 = true;
    d->scale_bf16 = present(a->scale) && a->scale.dtype == GMMFR_DT_BFLOAT16;
    d->pts_scalar = present(a->pertoken_scale) && a->pertoken_scale.dims[0] == 1;
    d->row_index_i32 = false;
  }
  return GMMFR_OK;
}

// Rules, in the order they are checked.  Operator rules cite
// "aclnnGroupedMatmulFinalizeRoutingWeightNzV2" (parameter notes, common
// constraints); the rest are this implementation's limits.
int validate(const gmmfr_args* a, Derived* d) {
  if (!a) return GMMFR_ERR_NULLPTR;
  // x1, x2, groupList are required; out is where the result goes.
  if (!present(a->x1) || !present(a->x2) || !present(a->group_list) || !present(a->out)) return GMMFR_ERR_NULLPTR;
  // reserved parameters must be null; bias placement is not specified
  if (present(a->bias) || present(a->offset) || present(a->antiquant_scale) || present(a->antiquant_offset))
    return GMMFR_ERR_UNSUPPORTED;
  if (present(a->scale) && a->scale.dtype == GMMFR_DT_INT64) return GMMFR_ERR_UNSUPPORTED;
  if (a->x1.dtype == GMMFR_DT_FLOAT8_E4M3FN)
    return a->x2.dtype == GMMFR_DT_FLOAT8_E4M3FN ? validate_fp8(a, d) : validate_mx(a, d);

  // element types
  if (a->x1.dtype != GMMFR_DT_INT8) return GMMFR_ERR_DTYPE;
  if (a->x2.dtype != GMMFR_DT_INT8 && a->x2.dtype != GMMFR_DT_INT32 && a->x2.dtype != GMMFR_DT_INT4) return GMMFR_ERR_DTYPE;
  if (present(a->scale) && a->scale.dtype != GMMFR_DT_FLOAT32 && a->scale.dtype != GMMFR_DT_BFLOAT16) return GMMFR_ERR_DTYPE;
  if (present(a->pertoken_scale) && a->pertoken_scale.dtype != GMMFR_DT_FLOAT32) return GMMFR_ERR_DTYPE;
  if (a->group_list.dtype != GMMFR_DT_INT64) return GMMFR_ERR_DTYPE;
  if (present(a->shared_input) && a->shared_input.dtype != GMMFR_DT_BFLOAT16) return GMMFR_ERR_DTYPE;
  if (present(a->logit) && a->logit.dtype != GMMFR_DT_FLOAT32) return GMMFR_ERR_DTYPE;
  if (present(a->row_index) && a->row_index.dtype != GMMFR_DT_INT64 && a->row_index.dtype != GMMFR_DT_INT32)
    return GMMFR_ERR_DTYPE;
  if (a->out.dtype != GMMFR_DT_FLOAT32) return GMMFR_ERR_DTYPE;
  if (present(a->acc_out) && a->acc_out.dtype != GMMFR_DT_INT32) return GMMFR_ERR_DTYPE;

  // attributes
  if (const int st = check_attributes(a)) return st;
  if (a->transpose_x1 != 0) return GMMFR_ERR_ATTR;
  if (a->transpose_x2 != 0 && a->transpose_x2 != 1) return GMMFR_ERR_ATTR;
  // transposed weights: (e,n,k) int8 (parameter notes: x2 (e,k,n), or (e,n,k)
  // when transposed); the int4 form is only given untransposed here
  const bool trans_b = a->transpose_x2 == 1;
  if (trans_b && a->x2.dtype != GMMFR_DT_INT8) return GMMFR_ERR_UNSUPPORTED;

  // shapes
  if (a->x1.ndim != 2) return GMMFR_ERR_SHAPE;
  const int64_t m = a->x1.dims[0], k = a->x1.dims[1];
  if (a->x2.ndim != 3) return GMMFR_ERR_SHAPE;
  const int64_t e = a->x2.dims[0];
  int64_t n;
  if (trans_b) n = a->x2.dims[1];
  else if (a->x2.dtype == GMMFR_DT_INT32) n = a->x2.dims[2] * 8;
  else n = a->x2.dims[2];
  const bool int4 = a->x2.dtype != GMMFR_DT_INT8;
  if (a->x2.dims[trans_b ? 2 : 1] != k) return GMMFR_ERR_SHAPE;
  if (m < 0 || m >= (int64_t(1) << 31)) return GMMFR_ERR_SHAPE;
  if (e < 1 || e > kMaxExperts) return GMMFR_ERR_SHAPE;
  if (k < 64 || k > 65536 || k % 64 != 0) return GMMFR_ERR_SHAPE;
  if (n < 16 || n % 16 != 0 || (int4 && n % 32 != 0)) return GMMFR_ERR_SHAPE;
  if (n > (int64_t(1) << 24) || m * n >= (int64_t(1) << 40)) return GMMFR_ERR_SHAPE;
  if (present(a->scale) && !dims_are(a->scale, 3, e, 1, n)) return GMMFR_ERR_SHAPE;
  // pertokenScale (m) per token, or (1): the static per-tensor activation
  // scale (function description: Atlas 350 static pertensor-perchannel)
  if (present(a->pertoken_scale) && !dims_are(a->pertoken_scale, 1, m) && !dims_are(a->pertoken_scale, 1, 1))
    return GMMFR_ERR_SHAPE;
  if (!dims_are(a->group_list, 1, e)) return GMMFR_ERR_SHAPE;
  if (present(a->logit) && !dims_are(a->logit, 1, m)) return GMMFR_ERR_SHAPE;
  if (present(a->row_index) && !dims_are(a->row_index, 1, m)) return GMMFR_ERR_SHAPE;
  if (present(a->acc_out) && !dims_are(a->acc_out, 2, m, n)) return GMMFR_ERR_SHAPE;
  int64_t bsdp = 0;
  if (const int st = check_output_and_alignment(a, n, &bsdp)) return st;
  const int64_t obs = a->output_bs;

  if (d) {
    d->m = m;
    d->k = k;
    d->n = n;
    d->e = e;
    d->bsdp = bsdp;
    d->output_bs = obs;
    d->int4 = int4;
    d->trans_b = trans_b;
    d->mx = false;
    d->fp8 = false;
    d->scale_bf16 = present(a->scale) && a->scale.dtype == GMMFR_DT_BFLOAT16;
    d->pts_scalar = present(a->pertoken_scale) && a->pertoken_scale.dims[0] == 1;
    d->row_index_i32 = present(a->row_index) && a->row_index.dtype == GMMFR_DT_INT32;
  }
  return GMMFR_OK;
}

// Tile choice from the expected rows per expert: tuningConfig[0] when given
// (the operator's tiling hint), else m / e.  Results do not depend on it.
TileId choose_tile(const gmmfr_args* a, const Derived& d, int cu_count) {
  int64_t expect = (d.m + d.e - 1) / d.e;
  if (a->tuning_config_len > 0 && a->tuning_config[0] > 0) expect = a->tuning_config[0];
  const int64_t ntn = (d.n + 255) / 256;
  // enough 256-row tiles for every CU to run several
  const bool big_ok = expect >= 1024 && (d.m / 256) * ntn >= 8 * (int64_t)std::max(cu_count, 1);
  if (d.mx || d.fp8) {  // the FP8 GEMMs: 256 x 256 (eight waves) or 128 x 256
    // Measured on the prefill shape: FP8 -3% (weights (e,k,n)) and -8%
    // ((e,n,k)) with the 256-row tile; MxA8W4 +0.5%, so it keeps 128 rows.
    const int64_t hint = a->tuning_config_len > 1 ? a->tuning_config[1] : 0;
    if (hint == 256 || (hint == 0 && big_ok && d.fp8))
      return (d.fp8 && d.k % 128 == 0) ? kTileFp8x256k128 : kTileMx256;
    return kTile128x256;
  }
  // The 256-row tile copies 128 k per stage (two stages) where it can: int8
  // weights and k % 128 == 0 (-2.6% GEMM time against 64 k per stage, four
  // stages, on the prefill shape); 64 k otherwise.
  const TileId big = (!d.int4 && d.k % 128 == 0) ? kTile256x256 : kTile256x256k64;
  // With int4 weights the 128-row tile copies 128 k per stage (two stages;
  // packed weights leave room for two workgroups per CU) when k % 128 == 0:
  // -8% GEMM time on the int4 workload against 64 k in three stages.
  const TileId mid = (d.int4 && d.k % 128 == 0) ? kTile128x256i4 : kTile128x256;
  if (a->tuning_config_len > 1) {  // explicit tile height
    switch (a->tuning_config[1]) {
      case 256: return big;
      case 128: return mid;
      case 64: return kTile64x256;
      case 32: return kTile32x256;
      default: break;
    }
  }
  // The 256-row tile (eight waves, one workgroup per CU) copies a third less
  // data per MAC than two 128-row tiles.  Measured GEMM times on MI355X, 32
  // experts of about 4096 rows, k = 2048, n = 7168: -6% with int8 weights
  // given (e,k,n), -15% given (e,n,k), but +4% with int4 weights; and +54%
  // with 512-row experts (8 experts, 4096 rows), where too few tiles reach
  // the 256 CUs.
  if (big_ok && !d.int4) return big;
  if (expect >= 256) return mid;
  if (expect >= 64) return kTile64x256;
  return kTile32x256;
}

// Rates measured on MI355X for the cost model below (both combine modes timed
// on every named workload on one box): fp32 atomics from the epilogue retire
// at about 1.3 TB/s of payload; the grouped GEMM runs at about
// 1.7 POP/s (int8, FP8 and MX) or 1.55 POP/s (int4 weights), or streams its
// weights at about 5 TB/s when each expert has few rows; the ordered reduce
// moves its bytes at about 5.4 TB/s.
constexpr double kAtomicBytesPerSec = 1.3e12;
constexpr double kGemmOpsPerSec = 1.7e15, kGemmOpsPerSecInt4 = 1.55e15;
constexpr double kWeightBytesPerSec = 5.0e12;
constexpr double kReduceBytesPerSec = 5.4e12;
constexpr double kOrderedLaunchScan = 8e-6, kOrderedLaunchBuckets = 25e-6;  // extra launches and their gaps

bool scan_lookup(const gmmfr_args* a, const Derived& d) {
  const int64_t lookup = a->tuning_config_len > 3 ? a->tuning_config[3] : 0;
  return lookup == 2 || (lookup == 0 && d.m * d.output_bs <= kScanReduceMax);
}

// Whether the hybrid combine is available: AUTO, int8 or int4 weights, and a
// tile whose continuous copy pipeline is compiled with it runs at this k.
bool hybrid_eligible(const gmmfr_args* a, const Derived& d, TileId tile) {
  if (a->deterministic == 1 || a->combine != GMMFR_COMBINE_AUTO || d.mx || d.fp8) return false;
  const TileShape ts = tile_shape(tile);
  return hybrid_compiled(tile) && uses_continuous_pipeline(d.int4, d.k, ts.bm, ts.bk, tile_stages(tile));
}

Combine choose_combine(const gmmfr_args* a, const Derived& d, TileId tile, int32_t* hybrid_atomic) {
  *hybrid_atomic = 0;
  if (a->deterministic == 1 || a->combine == GMMFR_COMBINE_ORDERED) return kCombineOrdered;
  if (a->combine == GMMFR_COMBINE_ATOMIC) return kCombineAtomic;
  const bool hyb_ok = hybrid_eligible(a, d, tile);
  if (hyb_ok && a->tuning_config_len > 4 && a->tuning_config[4] > 0) {
    *hybrid_atomic = (int32_t)a->tuning_config[4];
    return kCombineHybrid;
  }
  // From the shapes alone (the plan never reads device data).  Atomics
  // overlap the GEMM but slow it once they take more than about half of its
  // own time; the ordered path adds the reduce (contributions read once,
  // the output written once, sharedInput read) and its launches.
  const double contributions = (double)d.m * (double)d.n;
  const double t_atomic = contributions * 4.0 / kAtomicBytesPerSec;
  const double t_mfma = 2.0 * (double)d.m * (double)d.k * (double)d.n / (d.int4 ? kGemmOpsPerSecInt4 : kGemmOpsPerSec);
  const double experts = (double)std::min<int64_t>(d.e, std::max<int64_t>(d.m, 1));
  const double t_weights = experts * (double)d.k * (double)d.n * (d.int4 ? 0.5 : 1.0) / kWeightBytesPerSec;
  const double t_gemm = std::max(t_mfma, t_weights);
  const double reduce_bytes = contributions * 4.0 + (double)d.output_bs * (double)d.n * 4.0 + (double)d.bsdp * (double)d.n * 2.0;
  const double t_ordered_extra =
      reduce_bytes / kReduceBytesPerSec + (scan_lookup(a, d) ? kOrderedLaunchScan : kOrderedLaunchBuckets);
  return t_atomic <= 0.5 * t_gemm + t_ordered_extra ? kCombineAtomic : kCombineOrdered;
}

int make_plan(const gmmfr_args* a, const Derived& d, int cu_count, Plan* plan) {
  plan->tile = choose_tile(a, d, cu_count);
  const TileShape ts = tile_shape(plan->tile);
  plan->combine = choose_combine(a, d, plan->tile, &plan->hybrid_atomic);
  const int64_t ntn = (d.n + ts.bn - 1) / ts.bn;
  const int64_t max_tiles = ((d.m + ts.bm - 1) / ts.bm + d.e) * ntn;
  if (max_tiles >= (int64_t(1) << 31)) return GMMFR_ERR_SHAPE;
  const int64_t resident = (int64_t)std::max(cu_count, 1) * tile_occupancy(plan->tile);
  int64_t grid = std::min(max_tiles, resident);
  if (grid > 8) grid -= grid % 8;  // whole XCD rounds: workgroups are dealt to the 8 XCDs in turn
  // An explicit cap (tuningConfig[2], for tests: it makes every workgroup
  // run many tiles in a row) is taken as given, rounded or not.
  if (a->tuning_config_len > 2 && a->tuning_config[2] > 0) grid = std::min(grid, a->tuning_config[2]);
  plan->grid = d.m > 0 ? (int32_t)grid : 0;
  const bool ordered = plan->combine != kCombineAtomic;  // y and the ordered reduce (also hybrid)
  plan->scan_reduce = ordered && scan_lookup(a, d);
  const MxPad mp = mx_pad(d.mx, d.m, d.k, d.n, d.e);
  plan->workspace_bytes = workspace_layout(d.m, d.n, d.output_bs, ordered, mp.a_bytes, mp.b_bytes).total;
  return GMMFR_OK;
}

LaunchArgs to_launch(const gmmfr_args* a, const Derived& d) {
  LaunchArgs l;
  l.x1 = (const int8_t*)a->x1.data;
  l.x2 = a->x2.data;
  l.scale = a->scale.data;
  l.pertoken = (const float*)a->pertoken_scale.data;
  l.logit = (const float*)a->logit.data;
  l.group_list = (const int64_t*)a->group_list.data;
  l.row_index = a->row_index.data;
  l.shared = (const uint16_t*)a->shared_input.data;
  l.out = (float*)a->out.data;
  l.acc_out = (int32_t*)a->acc_out.data;
  l.m = d.m;
  l.k = d.k;
  l.n = d.n;
  l.e = (int32_t)d.e;
  l.group_list_type = (int32_t)a->group_list_type;
  l.scale_bf16 = d.scale_bf16;
  l.pertoken_scalar = d.pts_scalar;
  l.row_index_i32 = d.row_index_i32;
  l.int4 = d.int4;
  l.trans_b = d.trans_b;
  l.mx = d.mx;
  l.fp8 = d.fp8;
  l.bsdp = d.bsdp;
  l.shared_offset = present(a->shared_input) ? a->shared_input_offset : 0;
  l.output_bs = d.output_bs;
  return l;
}

int device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus;
}

bool log_enabled() {
  const char* v = std::getenv("GMMFR_LOG");
  return v && v[0] == '1';
}

// ---------------------------------------------------------------------------
// Scratch memory of the allocation-free entry point: one file-scope device
// array, GMMFR_NOALLOC_SCRATCH_BYTES long, which every GPU the library runs on
// holds until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and only that
// address is handed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[GMMFR_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on its
// first use there).  Returns GMMFR_OK or GMMFR_ERR_HIP.
int scratch_of_current_device(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GMMFR_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GMMFR_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return GMMFR_OK;
}

}  // namespace

extern "C" {

int gmm_finalize_routing_workspace(const gmmfr_args* args, size_t* workspace_bytes) {
  if (!workspace_bytes) return GMMFR_ERR_NULLPTR;
  Derived d;
  int st = validate(args, &d);
  if (st != GMMFR_OK) return st;
  Plan plan;
  st = make_plan(args, d, 1, &plan);
  if (st != GMMFR_OK) return st;
  *workspace_bytes = plan.workspace_bytes;
  return GMMFR_OK;
}

static int run_stage2(const gmmfr_args* args, void* workspace, size_t workspace_bytes, void* stream,
                      void* const* gemm_events) {
  Derived d;
  int st = validate(args, &d);
  if (st != GMMFR_OK) return st;
  Plan plan;
  st = make_plan(args, d, 1, &plan);  // workspace size does not depend on the device
  if (st != GMMFR_OK) return st;
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes)) return GMMFR_ERR_WORKSPACE;
  if (plan.workspace_bytes > 0 && !aligned16(workspace)) return GMMFR_ERR_ALIGN;
  const int cus = device_cu_count();
  if (cus <= 0) return GMMFR_ERR_HIP;
  st = make_plan(args, d, cus, &plan);
  if (st != GMMFR_OK) return st;
  if (log_enabled())
    std::fprintf(stderr, "[gmmfr] m=%lld k=%lld n=%lld e=%lld combine=%s(%d) %s grid=%d ws=%zu\n", (long long)d.m,
                 (long long)d.k, (long long)d.n, (long long)d.e,
                 plan.combine == kCombineOrdered ? "ordered" : plan.combine == kCombineHybrid ? "hybrid" : "atomic",
                 plan.hybrid_atomic,
                 tile_kernel_name(plan.tile, d.int4, d.k, d.trans_b, d.mx, d.fp8), plan.grid, plan.workspace_bytes);
  const int err = launch_all(to_launch(args, d), plan, workspace, stream, gemm_events);
  return err == 0 ? GMMFR_OK : GMMFR_ERR_HIP;
}

int gmm_finalize_routing(const gmmfr_args* args, void* workspace, size_t workspace_bytes, void* stream) {
  return run_stage2(args, workspace, workspace_bytes, stream, nullptr);
}

int gmm_finalize_routing_profiled(const gmmfr_args* args, void* workspace, size_t workspace_bytes, void* stream,
                                  void* gemm_start, void* gemm_stop) {
  void* ev[2] = {gemm_start, gemm_stop};
  return run_stage2(args, workspace, workspace_bytes, stream, ev);
}

int gmm_finalize_routing_noalloc(const gmmfr_args* args, void* stream) {
  // Validate and size on the host first: a plan that needs more scratch than
  // the array holds is rejected before any device is touched.
  Derived d;
  int st = validate(args, &d);
  if (st != GMMFR_OK) return st;
  Plan plan;
  st = make_plan(args, d, 1, &plan);
  if (st != GMMFR_OK) return st;
  if (plan.workspace_bytes > (size_t)GMMFR_NOALLOC_SCRATCH_BYTES) return GMMFR_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != GMMFR_OK) return st;
  return run_stage2(args, ws, (size_t)GMMFR_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int gmm_finalize_routing_plan(const gmmfr_args* args, gmmfr_plan_info* info) {
  if (!info) return GMMFR_ERR_NULLPTR;
  Derived d;
  int st = validate(args, &d);
  if (st != GMMFR_OK) return st;
  Plan plan;
  st = make_plan(args, d, 256, &plan);
  if (st != GMMFR_OK) return st;
  const TileShape ts = tile_shape(plan.tile);
  std::memset(info, 0, sizeof(*info));
  info->combine = plan.combine == kCombineOrdered  ? GMMFR_COMBINE_ORDERED
                  : plan.combine == kCombineHybrid ? GMMFR_COMBINE_HYBRID
                                                   : GMMFR_COMBINE_ATOMIC;
  info->hybrid_atomic = plan.combine == kCombineHybrid ? plan.hybrid_atomic : 0;
  info->tile_m = ts.bm;
  info->tile_n = ts.bn;
  info->tile_k = ts.bk;
  info->grid = plan.grid;
  info->int4_weights = d.int4 ? 1 : 0;
  info->workspace_bytes = (int64_t)plan.workspace_bytes;
  std::snprintf(info->gemm_kernel, sizeof(info->gemm_kernel), "%s", tile_kernel_name(plan.tile, d.int4, d.k, d.trans_b, d.mx, d.fp8));
  return GMMFR_OK;
}

const char* gmmfr_status_string(int status) {
  switch (status) {
    case GMMFR_OK: return "ok";
    case GMMFR_ERR_NULLPTR: return "null pointer";
    case GMMFR_ERR_DTYPE: return "unsupported element type";
    case GMMFR_ERR_SHAPE: return "inconsistent or unsupported shape";
    case GMMFR_ERR_ATTR: return "invalid attribute";
    case GMMFR_ERR_UNSUPPORTED: return "unsupported optional input";
    case GMMFR_ERR_ALIGN: return "misaligned pointer";
    case GMMFR_ERR_WORKSPACE: return "workspace missing or too small";
    case GMMFR_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

}  // extern "C"
