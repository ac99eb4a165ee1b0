// Producer step of the grouped matmul: dynamic per-token int8 quantisation of
// bf16 hidden states and the routing permute (x1, pertokenScale, logit,
// rowIndex and groupList from a router's top-K choice).
//
// The pages name the step without its formulas: a permute after the dispatch
// and before the expert matmul, and a per-token dynamic quantisation mode
// ("aclnnAlltoAllvQuantGroupedMatMul", function and formula; quantisation
// modes); the per-token cast multiplies by an inverse scale (PTOAS issue
// #1568, background).  Reading taken (plain symmetric int8):
//   amax = max |x|, scale = fl(amax / 127), inv = fl(127 / amax) (0 if amax = 0),
//   q = clamp(rne(fl(x * inv)), -127, 127);
//   rows = local (token, slot) entries sorted by local expert, ties in
//   ascending entry index t*K + j.
//
// Kernels, in stream order:
//   route_count_kernel    entries per (local expert, chunk of 256 entries)
//   route_expert_scan_kernel  one workgroup per expert: its rows before each
//                         chunk, and its total
//   route_scatter_kernel  expert totals scanned in every workgroup (the first
//                         row of each expert; groupList); stable rank of
//                         every entry inside its chunk (one
//                         wave per chunk, 64 entries per step, peers found by
//                         matching expert bits across the wave) -> its row;
//                         writes rowIndex, logit and the entry -> row map
//   quant_rows_kernel     one wave per token: amax, scale, then the int8 row
//                         written to each of the token's rows
// All HBM-bound; the quantisation moves T*k*2 bytes in and T*K*k bytes out.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "../../include/gmmfr.h"

namespace gmmqp {

constexpr int kQpThreads = 256;
constexpr int kQpWaves = kQpThreads / 64;
constexpr int kRouteChunk = 256;       // entries per wave in the routing kernels
constexpr int kMaxLocalExperts = 1024;
constexpr int kMaxTopK = 64;           // one lane per slot of a token
constexpr int kQuantCols = 16;         // bf16 values per lane per step

struct QpParams {
  const uint16_t* hidden;   // (T,k) bf16 bits
  const void* ids;          // (T,K) int32 or int64
  const float* weights;     // (T,K) or nullptr
  int8_t* x1;               // (T*K,k)
  float* pts;               // (T*K)
  float* logit;             // (T*K) or nullptr
  void* row_index;          // (T*K) int32 or int64
  int64_t* group_list;      // (e)
  int32_t* chunk_base;      // (e, nchunks): counts, then the first row of each (expert, chunk)
  int32_t* pos_of;          // (T*K): row of each entry, -1 when it is not local
  int64_t T, k, nflat, offset;
  int32_t K, e, nchunks, ids_i32, ri_i32, glt;
};

// x1 encodings of the quantisation step
constexpr int kQInt8 = 0;  // int8 per token, pertokenScale fp32 (m)
constexpr int kQFp8 = 1;   // FP8 E4M3 per token, pertokenScale fp32 (m)
constexpr int kQMx = 2;    // FP8 E4M3 with one E8M0 scale per 32 values, pertokenScale (m, k/64, 2)

// Local expert of entry f, or -1 when its id lies outside [offset, offset+e)
// (unsigned difference: no overflow for any id).
__device__ __forceinline__ int local_expert(const QpParams& q, int64_t f) {
  const int64_t id = q.ids_i32 ? (int64_t)((const int32_t*)q.ids)[f] : ((const int64_t*)q.ids)[f];
  const uint64_t g = (uint64_t)id - (uint64_t)q.offset;
  return g < (uint64_t)q.e ? (int)g : -1;
}

__global__ __launch_bounds__(kQpThreads) void route_count_kernel(QpParams q) {
  __shared__ int32_t s_cnt[kQpWaves][kMaxLocalExperts];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * kQpWaves + w;
  for (int g = lane; g < q.e; g += 64) s_cnt[w][g] = 0;
  __syncthreads();
  if (c < q.nchunks) {
    const int64_t f0 = (int64_t)c * kRouteChunk;
    for (int it = 0; it < kRouteChunk / 64; ++it) {
      const int64_t f = f0 + it * 64 + lane;
      if (f < q.nflat) {
        const int g = local_expert(q, f);
        if (g >= 0) atomicAdd(&s_cnt[w][g], 1);
      }
    }
  }
  __syncthreads();
  if (c < q.nchunks)
    for (int g = lane; g < q.e; g += 64) q.chunk_base[(int64_t)g * q.nchunks + c] = s_cnt[w][g];
}

// Exclusive scan of s[0..n) in place, n <= 4 * kQpThreads, by the whole
// workgroup (kQpThreads threads, four values each); returns the total.
// s_tmp holds kQpThreads values.  Ends with a barrier.
__device__ int32_t block_exclusive_scan(int32_t* s, int n, int32_t* s_tmp) {
  const int t = threadIdx.x;
  int32_t v[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = t * 4 + i < n ? s[t * 4 + i] : 0;
    sum += v[i];
  }
  s_tmp[t] = sum;
  __syncthreads();
  for (int off = 1; off < kQpThreads; off <<= 1) {
    const int32_t x = t >= off ? s_tmp[t - off] : 0;
    __syncthreads();
    s_tmp[t] += x;
    __syncthreads();
  }
  int32_t run = s_tmp[t] - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (t * 4 + i < n) s[t * 4 + i] = run;
    run += v[i];
  }
  const int32_t total = s_tmp[kQpThreads - 1];
  __syncthreads();
  return total;
}

// One workgroup per local expert g: its chunk counts become exclusive
// prefixes in place (the expert's rows before each chunk) and its total goes
// to totals[g].  Each thread takes a contiguous run of chunks.
__global__ __launch_bounds__(kQpThreads) void route_expert_scan_kernel(QpParams q, int32_t* totals) {
  __shared__ int32_t s_sum[kQpThreads * 4];
  __shared__ int32_t s_tmp[kQpThreads];
  const int g = blockIdx.x, t = threadIdx.x;
  int32_t* row = q.chunk_base + (int64_t)g * q.nchunks;
  const int len = (q.nchunks + kQpThreads - 1) / kQpThreads;
  const int c0 = min(t * len, q.nchunks), c1 = min(c0 + len, q.nchunks);
  constexpr int kBatch = 16;  // loads in independent batches (one memory round trip each)
  int32_t sum = 0;
  for (int c = c0; c < c1; c += kBatch) {
    int32_t v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) v[i] = c + i < c1 ? row[c + i] : 0;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) sum += v[i];
  }
  s_sum[t] = sum;
  __syncthreads();
  const int32_t total = block_exclusive_scan(s_sum, kQpThreads, s_tmp);
  int32_t run = s_sum[t];
  for (int c = c0; c < c1; c += kBatch) {
    int32_t v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) v[i] = c + i < c1 ? row[c + i] : 0;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (c + i < c1) {
        row[c + i] = run;
        run += v[i];
      }
  }
  if (t == 0) totals[g] = total;
}

// Each workgroup first scans the expert totals (the first row of every
// expert); workgroup 0 also writes groupList from them.
__global__ __launch_bounds__(kQpThreads) void route_scatter_kernel(QpParams q, const int32_t* totals) {
  __shared__ int32_t s_run[kQpWaves][kMaxLocalExperts];
  __shared__ int32_t s_start[kMaxLocalExperts];
  __shared__ int32_t s_tmp[kQpThreads];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = blockIdx.x * kQpWaves + w;
  for (int g = threadIdx.x; g < q.e; g += kQpThreads) s_start[g] = totals[g];
  __syncthreads();
  block_exclusive_scan(s_start, q.e, s_tmp);
  if (blockIdx.x == 0)
    for (int g = threadIdx.x; g < q.e; g += kQpThreads)
      q.group_list[g] = q.glt == 1 ? (int64_t)totals[g] : (int64_t)s_start[g] + totals[g];
  if (c < q.nchunks)
    for (int g = lane; g < q.e; g += 64) s_run[w][g] = s_start[g] + q.chunk_base[(int64_t)g * q.nchunks + c];
  __syncthreads();
  if (c >= q.nchunks) return;  // wave-uniform; no barrier follows
  const int bits = 32 - __clz(q.e);  // keys g + 1 lie in [0, e]
  const uint64_t below = (1ull << lane) - 1;
  const int64_t f0 = (int64_t)c * kRouteChunk;
  for (int it = 0; it < kRouteChunk / 64; ++it) {
    const int64_t f = f0 + it * 64 + lane;
    const bool in = f < q.nflat;
    const int g = in ? local_expert(q, f) : -1;
    // lanes holding the same key (all 64 lanes take part in every ballot)
    const unsigned key = (unsigned)(g + 1);
    uint64_t peers = ~0ull;
    for (int b = 0; b < bits; ++b) {
      const uint64_t set = __ballot((key >> b) & 1u);
      peers &= ((key >> b) & 1u) ? set : ~set;
    }
    int pos = -1;
    if (g >= 0) pos = s_run[w][g] + __popcll(peers & below);
    // every lane's read above precedes the leader's update below (one wave's
    // LDS operations execute in program order)
    if (g >= 0 && (peers & below) == 0) s_run[w][g] += __popcll(peers);
    if (in) q.pos_of[f] = pos;
    if (pos >= 0) {
      const int64_t t = f / q.K;
      if (q.ri_i32) ((int32_t*)q.row_index)[pos] = (int32_t)t;
      else ((int64_t*)q.row_index)[pos] = t;
      if (q.weights) q.logit[pos] = q.weights[f];
    }
  }
}

__device__ __forceinline__ float bf16f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t quant4(uint32_t lo2, uint32_t hi2, float inv) {
  // four bf16 (two per word, low half first) -> four int8 codes, low byte first
  const float v[4] = {bf16f(lo2 & 0xFFFFu), bf16f(lo2 >> 16), bf16f(hi2 & 0xFFFFu), bf16f(hi2 >> 16)};
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float r = __builtin_rintf(__fmul_rn(v[i], inv));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    out |= ((uint32_t)(int32_t)r & 0xFFu) << (8 * i);
  }
  return out;
}

// fp32 -> FP8 E4M3 code for |v| <= 448 (the caller saturates): round to
// nearest, ties to even.  Normal range: keep 3 mantissa bits of the binary32
// pattern, rounding the 20 dropped ones to nearest even (a carry moves into
// the exponent), and rebias the exponent from 127 to 7; below 2^-6 the
// subnormal grid of 2^-9.
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {
    code = (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8; 8 is the smallest normal's code
  } else {
    const uint32_t ab = bits & 0x7FFFFFFFu;
    const uint32_t r = ab + 0x7FFFFu + ((ab >> 20) & 1u);
    code = (r >> 20) - ((127u - 7u) << 3);
  }
  return sign | code;
}

// One wave per token.  NI > 0: the row has at most NI*1024 values and stays in
// registers between the amax pass and the quantisation; NI = 0: any k, the
// second pass reads the row again (from cache).  QM: the x1 encoding.  For MX
// the two lanes holding a 32-value block (16 values each) share its maximum.
template <int NI, int QM>
__global__ __launch_bounds__(kQpThreads) void quant_rows_kernel(QpParams q) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  constexpr int kStep = 64 * kQuantCols;
  for (int64_t t = (int64_t)blockIdx.x * kQpWaves + w; t < q.T; t += (int64_t)gridDim.x * kQpWaves) {
    const uint16_t* row = q.hidden + t * q.k;
    const int32_t dst = lane < q.K ? q.pos_of[t * q.K + lane] : -1;
    constexpr int NR = NI > 0 ? NI : 1;
    uint4 a[NR], b[NR];
    // |x| of a finite bf16 orders like its 15 low bits
    uint32_t mag = 0;
    auto fold = [&](const uint4& u, const uint4& v) {
      const uint32_t wv[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) mag = max(mag, max(wv[i] & 0x7FFFu, (wv[i] >> 16) & 0x7FFFu));
    };
    if constexpr (NI > 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int64_t c = (int64_t)lane * kQuantCols + i * kStep;
        a[i] = make_uint4(0, 0, 0, 0);
        b[i] = a[i];
        if (c < q.k) {
          a[i] = *(const uint4*)(row + c);
          b[i] = *(const uint4*)(row + c + 8);
        }
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) fold(a[i], b[i]);
    } else {
      for (int64_t c = (int64_t)lane * kQuantCols; c < q.k; c += kStep)
        fold(*(const uint4*)(row + c), *(const uint4*)(row + c + 8));
    }
    float inv = 0.0f;
    if constexpr (QM != kQMx) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) mag = max(mag, (uint32_t)__shfl_xor((int)mag, off));
      const float amax = bf16f(mag);
      const float top = QM == kQInt8 ? 127.0f : 448.0f;  // the largest code magnitude
      const float scale = __fdiv_rn(amax, top);
      inv = amax > 0.0f ? __fdiv_rn(top, amax) : 0.0f;
      if (dst >= 0) q.pts[dst] = scale;
    }
    // x1 rows are written once and not read again here: nontemporal stores
    // (measured 16% faster for the whole step than plain stores)
    auto emit = [&](int64_t c, const uint4& u, const uint4& v) {
      u32x4 o;
      if constexpr (QM == kQInt8) {
        o = u32x4{quant4(u.x, u.y, inv), quant4(u.z, u.w, inv), quant4(v.x, v.y, inv), quant4(v.z, v.w, inv)};
      } else {
        // FP8 per token: codes of fl(x * inv), saturated to +-448.  MX: the
        // block's shared exponent from its largest magnitude's bf16 exponent
        // field E (floor(log2) - 8, clamped at -127: E8M0 code max(E - 8, 0)),
        // codes of x * 2^(127 - code), saturated.
        int shift = 0;
        uint32_t bcode = 0;
        if constexpr (QM == kQMx) {
          uint32_t bm = 0;
          const uint32_t wv[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) bm = max(bm, max(wv[i] & 0x7FFFu, (wv[i] >> 16) & 0x7FFFu));
          bm = max(bm, (uint32_t)__shfl_xor((int)bm, 1));
          const uint32_t ex = bm >> 7;
          bcode = ex >= 8 ? ex - 8 : 0;
          shift = 127 - (int)bcode;
        }
        auto enc4 = [&](uint32_t lo2, uint32_t hi2) {
          const float x[4] = {bf16f(lo2 & 0xFFFFu), bf16f(lo2 >> 16), bf16f(hi2 & 0xFFFFu), bf16f(hi2 >> 16)};
          uint32_t w = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float t = QM == kQMx ? ldexpf(x[i], shift) : __fmul_rn(x[i], inv);
            w |= e4m3_code(fminf(fmaxf(t, -448.0f), 448.0f)) << (8 * i);
          }
          return w;
        };
        o = u32x4{enc4(u.x, u.y), enc4(u.z, u.w), enc4(v.x, v.y), enc4(v.z, v.w)};
        if constexpr (QM == kQMx) {
          // the even lane of the pair writes the block's E8M0 code to each row
          if ((lane & 1) == 0) {
            for (int j = 0; j < q.K; ++j) {
              const int32_t d = __builtin_amdgcn_readlane(dst, j);
              if (d >= 0) ((uint8_t*)q.pts)[(int64_t)d * (q.k / 32) + c / 32] = (uint8_t)bcode;
            }
          }
        }
      }
      for (int j = 0; j < q.K; ++j) {
        const int32_t d = __builtin_amdgcn_readlane(dst, j);
        if (d >= 0) __builtin_nontemporal_store(o, (u32x4*)(q.x1 + (int64_t)d * q.k + c));
      }
    };
    if constexpr (NI > 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int64_t c = (int64_t)lane * kQuantCols + i * kStep;
        if (c < q.k) emit(c, a[i], b[i]);
      }
    } else {
      for (int64_t c = (int64_t)lane * kQuantCols; c < q.k; c += kStep)
        emit(c, *(const uint4*)(row + c), *(const uint4*)(row + c + 8));
    }
  }
}

// ---------------------------------------------------------------- host side

bool given(const gmmfr_tensor& t) {
  if (t.data != nullptr) return true;
  for (int i = 0; i < t.ndim && i < 4; ++i)
    if (t.dims[i] == 0) return true;
  return false;
}

bool shape_is(const gmmfr_tensor& t, int nd, int64_t d0, int64_t d1 = -1) {
  if (t.ndim != nd) return false;
  if (t.dims[0] != d0) return false;
  return nd < 2 || t.dims[1] == d1;
}

size_t round256(size_t v) { return (v + 255) & ~size_t(255); }

struct QpPlan {
  int64_t T, k, nflat;
  int32_t K, e, nchunks, qmode;
  size_t base_off, tot_off, pos_off, total;
};

int qp_validate(const gmmqp_args* a, QpPlan* p) {
  if (!a) return GMMFR_ERR_NULLPTR;
  if (!given(a->hidden) || !given(a->expert_ids) || !given(a->x1) || !given(a->pertoken_scale) ||
      !given(a->row_index) || !given(a->group_list))
    return GMMFR_ERR_NULLPTR;
  if (given(a->topk_weights) != given(a->logit)) return GMMFR_ERR_NULLPTR;
  if (a->hidden.dtype != GMMFR_DT_BFLOAT16) return GMMFR_ERR_DTYPE;
  if (a->expert_ids.dtype != GMMFR_DT_INT32 && a->expert_ids.dtype != GMMFR_DT_INT64) return GMMFR_ERR_DTYPE;
  if (given(a->topk_weights) && a->topk_weights.dtype != GMMFR_DT_FLOAT32) return GMMFR_ERR_DTYPE;
  // x1 INT8 with FLOAT32 per-token scales; FLOAT8_E4M3FN with FLOAT32 per-token
  // scales, or with FLOAT8_E8M0 scales per 32 values (MX)
  int qmode;
  if (a->x1.dtype == GMMFR_DT_INT8 && a->pertoken_scale.dtype == GMMFR_DT_FLOAT32) qmode = kQInt8;
  else if (a->x1.dtype == GMMFR_DT_FLOAT8_E4M3FN && a->pertoken_scale.dtype == GMMFR_DT_FLOAT32) qmode = kQFp8;
  else if (a->x1.dtype == GMMFR_DT_FLOAT8_E4M3FN && a->pertoken_scale.dtype == GMMFR_DT_FLOAT8_E8M0) qmode = kQMx;
  else return GMMFR_ERR_DTYPE;
  if (given(a->logit) && a->logit.dtype != GMMFR_DT_FLOAT32) return GMMFR_ERR_DTYPE;
  if (a->row_index.dtype != GMMFR_DT_INT32 && a->row_index.dtype != GMMFR_DT_INT64) return GMMFR_ERR_DTYPE;
  if (a->group_list.dtype != GMMFR_DT_INT64) return GMMFR_ERR_DTYPE;
  if (a->group_list_type != 0 && a->group_list_type != 1) return GMMFR_ERR_ATTR;
  if (a->hidden.ndim != 2 || a->expert_ids.ndim != 2) return GMMFR_ERR_SHAPE;
  const int64_t T = a->hidden.dims[0], k = a->hidden.dims[1], K = a->expert_ids.dims[1];
  if (a->expert_ids.dims[0] != T || T < 0) return GMMFR_ERR_SHAPE;
  if (K < 1 || K > kMaxTopK) return GMMFR_ERR_SHAPE;
  if (k < kQuantCols || k > 65536 || k % kQuantCols != 0) return GMMFR_ERR_SHAPE;
  if (T > (int64_t(1) << 31) / K) return GMMFR_ERR_SHAPE;
  const int64_t m = T * K;
  if (m >= (int64_t(1) << 31)) return GMMFR_ERR_SHAPE;
  if (a->group_list.ndim != 1) return GMMFR_ERR_SHAPE;
  const int64_t e = a->group_list.dims[0];
  if (e < 1 || e > kMaxLocalExperts) return GMMFR_ERR_SHAPE;
  if (given(a->topk_weights) && !shape_is(a->topk_weights, 2, T, K)) return GMMFR_ERR_SHAPE;
  if (!shape_is(a->x1, 2, m, k) || !shape_is(a->row_index, 1, m)) return GMMFR_ERR_SHAPE;
  if (qmode == kQMx) {
    const gmmfr_tensor& t = a->pertoken_scale;  // (m, k/64, 2): one E8M0 per 32 values
    if (k % 64 != 0 || t.ndim != 3 || t.dims[0] != m || t.dims[1] != k / 64 || t.dims[2] != 2) return GMMFR_ERR_SHAPE;
  } else if (!shape_is(a->pertoken_scale, 1, m)) {
    return GMMFR_ERR_SHAPE;
  }
  if (given(a->logit) && !shape_is(a->logit, 1, m)) return GMMFR_ERR_SHAPE;
  const gmmfr_tensor* all[] = {&a->hidden, &a->expert_ids, &a->topk_weights, &a->x1, &a->pertoken_scale,
                               &a->logit, &a->row_index, &a->group_list};
  for (const gmmfr_tensor* t : all)
    if (given(*t) && ((uintptr_t)t->data & 15u) != 0) return GMMFR_ERR_ALIGN;
  if (p) {
    p->T = T;
    p->k = k;
    p->K = (int32_t)K;
    p->e = (int32_t)e;
    p->nflat = m;
    p->qmode = qmode;
    p->nchunks = (int32_t)((m + kRouteChunk - 1) / kRouteChunk);
    p->base_off = 0;
    p->tot_off = round256((size_t)e * p->nchunks * 4);
    p->pos_off = p->tot_off + round256((size_t)e * 4);
    p->total = p->pos_off + round256((size_t)m * 4);
  }
  return GMMFR_OK;
}

int qp_run(const gmmqp_args* a, void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
  QpPlan p;
  const int st = qp_validate(a, &p);
  if (st != GMMFR_OK) return st;
  if (p.total > 0 && (!workspace || workspace_bytes < p.total)) return GMMFR_ERR_WORKSPACE;
  if (p.total > 0 && ((uintptr_t)workspace & 15u) != 0) return GMMFR_ERR_ALIGN;
  QpParams q;
  q.hidden = (const uint16_t*)a->hidden.data;
  q.ids = a->expert_ids.data;
  q.weights = given(a->topk_weights) ? (const float*)a->topk_weights.data : nullptr;
  q.x1 = (int8_t*)a->x1.data;
  q.pts = (float*)a->pertoken_scale.data;
  q.logit = given(a->logit) ? (float*)a->logit.data : nullptr;
  q.row_index = a->row_index.data;
  q.group_list = (int64_t*)a->group_list.data;
  q.chunk_base = (int32_t*)((char*)workspace + p.base_off);
  q.pos_of = (int32_t*)((char*)workspace + p.pos_off);
  q.T = p.T;
  q.k = p.k;
  q.nflat = p.nflat;
  q.offset = a->expert_offset;
  q.K = p.K;
  q.e = p.e;
  q.nchunks = p.nchunks;
  q.ids_i32 = a->expert_ids.dtype == GMMFR_DT_INT32;
  q.ri_i32 = a->row_index.dtype == GMMFR_DT_INT32;
  q.glt = (int32_t)a->group_list_type;
  hipStream_t s = (hipStream_t)stream;
  const int rgrid = (p.nchunks + kQpWaves - 1) / kQpWaves;
  if (rgrid > 0) hipLaunchKernelGGL(route_count_kernel, dim3(rgrid), dim3(kQpThreads), 0, s, q);
  int32_t* totals = (int32_t*)((char*)workspace + p.tot_off);
  hipLaunchKernelGGL(route_expert_scan_kernel, dim3(p.e), dim3(kQpThreads), 0, s, q, totals);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(rgrid > 0 ? rgrid : 1), dim3(kQpThreads), 0, s, q,
                     (const int32_t*)totals);
  if (p.T > 0) {
    const int64_t want = (p.T + kQpWaves - 1) / kQpWaves;
    const int qgrid = (int)(want < 65536 ? want : 65536);
    if (events && events[0] && hipEventRecord((hipEvent_t)events[0], s) != hipSuccess) return GMMFR_ERR_HIP;
    auto launch = [&](auto qm_) {
      constexpr int QM = decltype(qm_)::value;
      if (p.k <= 1024) hipLaunchKernelGGL((quant_rows_kernel<1, QM>), dim3(qgrid), dim3(kQpThreads), 0, s, q);
      else if (p.k <= 2048) hipLaunchKernelGGL((quant_rows_kernel<2, QM>), dim3(qgrid), dim3(kQpThreads), 0, s, q);
      else if (p.k <= 4096) hipLaunchKernelGGL((quant_rows_kernel<4, QM>), dim3(qgrid), dim3(kQpThreads), 0, s, q);
      else hipLaunchKernelGGL((quant_rows_kernel<0, QM>), dim3(qgrid), dim3(kQpThreads), 0, s, q);
    };
    if (p.qmode == kQMx) launch(std::integral_constant<int, kQMx>{});
    else if (p.qmode == kQFp8) launch(std::integral_constant<int, kQFp8>{});
    else launch(std::integral_constant<int, kQInt8>{});
    if (events && events[1] && hipEventRecord((hipEvent_t)events[1], s) != hipSuccess) return GMMFR_ERR_HIP;
  }
  return hipGetLastError() == hipSuccess ? GMMFR_OK : GMMFR_ERR_HIP;
}

}  // namespace gmmqp

extern "C" {

using namespace gmmqp;

int gmm_quant_permute_workspace(const gmmqp_args* args, size_t* workspace_bytes) {
  QpPlan p;
  const int st = qp_validate(args, &p);
  if (st != GMMFR_OK) return st;
  if (!workspace_bytes) return GMMFR_ERR_NULLPTR;
  *workspace_bytes = p.total;
  return GMMFR_OK;
}

int gmm_quant_permute(const gmmqp_args* args, void* workspace, size_t workspace_bytes, void* stream) {
  return qp_run(args, workspace, workspace_bytes, stream, nullptr);
}

int gmm_quant_permute_profiled(const gmmqp_args* args, void* workspace, size_t workspace_bytes, void* stream,
                               void* quant_start, void* quant_stop) {
  void* ev[2] = {quant_start, quant_stop};
  return qp_run(args, workspace, workspace_bytes, stream, ev);
}

}  // extern "C"
