// HIP kernels for gfx950 (CDNA4): grouped int8 / int4 MFMA GEMM with fused
// dequantisation and finalize-routing combine.
//
// What is computed ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", function
// description and parameter notes; epilogue order from the worked example of
// "matmul支持pertoken量化模式"):
//   acc[i][j] = sum_kk x1[i][kk] * x2[g][kk][j]          (int32, exact)
//   y[i][j]   = ((float(acc) * scale[g][j]) * pts[i]) * logit[i]   (fp32)
//   out       = seed;  out[rowIndex[i]] += y[i]           (combine by index)
//
// Kernels
//   seed_kernel        out := 0, rows [off, off+bsdp) := widened sharedInput
//   gmm_kernel<...>    persistent grouped GEMM; epilogue adds into out with
//                      fp32 atomics, or stores y for the ordered combine
//   hist/scan/scatter  rows bucketed by destination (ordered combine)
//   reduce_kernel      per destination: sort its rows ascending, fold
//                      seed + y[rows] in that order, write out once
#include <hip/hip_runtime.h>

#include <algorithm>

#include "gmmfr_internal.h"

namespace gmmfr {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
#define LDS_PTR(T) __attribute__((address_space(3))) T*

constexpr int kThreads = 256;

struct KParams {
  const int8_t* x1;
  const void* x2;
  const void* scale;
  const float* pertoken;
  const float* logit;
  const int64_t* group_list;
  const void* row_index;
  const uint16_t* shared;
  float* out;
  float* y;             // ordered combine: (m,n) contributions
  int32_t* acc_out;
  int64_t m, k, n;
  int64_t bsdp, shared_offset, output_bs;
  int32_t e, group_list_type, scale_bf16, row_index_i32;
  int32_t n_tiles_n;
  int32_t combine;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Destination row of source row i; -1 when outside [0, output_bs).
__device__ __forceinline__ int64_t dest_row(const KParams& p, int64_t i) {
  int64_t d;
  if (!p.row_index) d = i;
  else if (p.row_index_i32) d = ((const int32_t*)p.row_index)[i];
  else d = ((const int64_t*)p.row_index)[i];
  return (d >= 0 && d < p.output_bs) ? d : -1;
}

// ---------------------------------------------------------------------------
// groupList -> per-expert row ranges and tile prefix, computed by every
// workgroup into LDS (e <= 1024).  Type 0 lists cumulative ends, type 1 lists
// counts ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", common constraints).
// Device data are not trusted: each entry is clamped to [0, m], ends are made
// non-decreasing (running max for type 0, running sum for type 1) and capped
// at m, so a broken list never leads outside x1.
// ---------------------------------------------------------------------------
__device__ void block_scan_i64(int64_t (&v)[kMaxExperts / kThreads], bool use_max, int64_t* s_scan) {
  constexpr int PER = kMaxExperts / kThreads;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 1; q < PER; ++q) v[q] = use_max ? max(v[q - 1], v[q]) : v[q - 1] + v[q];
  s_scan[tid] = v[PER - 1];
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    int64_t t = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] = use_max ? max(s_scan[tid], t) : s_scan[tid] + t;
    __syncthreads();
  }
  int64_t excl = tid > 0 ? s_scan[tid - 1] : 0;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < PER; ++q) v[q] = use_max ? max(excl, v[q]) : excl + v[q];
}

// s_ends[g] = end row of expert g; s_tile_pre[g] = first tile of expert g,
// s_tile_pre[e] = total tiles.
__device__ void build_group_table(const KParams& p, int bm, int32_t* s_ends, int32_t* s_tile_pre, int64_t* s_scan) {
  constexpr int PER = kMaxExperts / kThreads;
  const int tid = threadIdx.x;
  int64_t v[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = tid * PER + q;
    int64_t x = g < p.e ? p.group_list[g] : 0;
    v[q] = min(max(x, (int64_t)0), p.m);
  }
  block_scan_i64(v, p.group_list_type == 0, s_scan);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = tid * PER + q;
    if (g < p.e) s_ends[g] = (int32_t)min(v[q], p.m);
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = tid * PER + q;
    int64_t t = 0;
    if (g < p.e) {
      const int64_t c = s_ends[g] - (g ? s_ends[g - 1] : 0);
      t = ((c + bm - 1) / bm) * p.n_tiles_n;
    }
    v[q] = t;
  }
  block_scan_i64(v, false, s_scan);
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = tid * PER + q;
    if (g < p.e) s_tile_pre[g + 1] = (int32_t)v[q];
  }
  if (tid == 0) s_tile_pre[0] = 0;
  __syncthreads();
}

// Expert owning tile t: the largest g with s_tile_pre[g] <= t.
__device__ __forceinline__ int find_group(const int32_t* s_tile_pre, int e, int t) {
  int lo = 0, hi = e - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_tile_pre[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// LDS layouts (conflict-free for 128-byte bank windows):
//   A stage: [BM][BK] bytes, k-contiguous; 16-byte chunk c of row r is stored
//            at chunk position c ^ swz_a(r).  Read with ds_read_b128.
//   B stage: [BK][BN] bytes, n-contiguous (the weight's own layout); chunk c
//            of k-row r is stored at position c ^ (r & 7).  Read with the
//            gfx950 transpose load ds_read_b64_tr_b8: within each 16-lane
//            group, lane 16G+i receives byte (i % 8) of the eight 8-byte rows
//            addressed by lanes 16G + 2b + i/8 (b = 0..7).  Lane s therefore
//            supplies k-row (s%16)/2 at column 16*((s/16)%2) + 8*(s%2) and
//            gets eight consecutive k of column s%32; two such loads give the
//            16 k-values the i8 MFMA expects per lane.
// Both stages are filled by global_load_lds_dwordx4 (HBM -> LDS without
// VGPRs); a lane's LDS slot is fixed, so the swizzle is applied by choosing
// which global chunk each lane fetches.
// ---------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ int swz_a(int r) {
  if constexpr (BK == 64) return ((r >> 1) ^ (r >> 3)) & 3;
  else return (r ^ (r >> 3)) & 7;
}
__device__ __forceinline__ int swz_b(int r) { return r & 7; }

__device__ __forceinline__ void lds_dma16(const void* gsrc, LDS_PTR(void) ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, ldst, 16, 0, 0);
}

// int4 word -> 8 int8 holding 16 * value, in column order (two dwords).
__device__ __forceinline__ void unpack_int4_x16(uint32_t w, uint32_t& d0, uint32_t& d1) {
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u;  // 16*t0, 16*t2, 16*t4, 16*t6
  const uint32_t hi = w & 0xF0F0F0F0u;         // 16*t1, 16*t3, 16*t5, 16*t7
  d0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // t0 t1 t2 t3
  d1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // t4 t5 t6 t7
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int OCC, bool INT4>
__global__ __launch_bounds__(kThreads, OCC) void gmm_kernel(KParams p) {
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int CPR_A = BK / 16, CPR_B = BN / 16;
  constexpr int A_BYTES = BM * BK, B_BYTES = BK * BN;
  constexpr int A_SLOTS = BM * CPR_A, B_SLOTS = BK * CPR_B;
  constexpr int NWAVES = kThreads / 64;
  static_assert(WAVES_M * WAVES_N == NWAVES, "4 waves");
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(BN >= 128, "B swizzle needs 8 chunks per row");
  static_assert(A_SLOTS % 64 == 0 && B_SLOTS % 64 == 0, "whole waves per copy");

  __shared__ __attribute__((aligned(16))) int8_t smA[2 * A_BYTES];
  __shared__ __attribute__((aligned(16))) int8_t smB[2 * B_BYTES];
  __shared__ int32_t s_ends[kMaxExperts];
  __shared__ int32_t s_tile_pre[kMaxExperts + 1];
  __shared__ int64_t s_scan[kThreads];
  __shared__ float s_pts[BM], s_logit[BM];
  __shared__ int32_t s_dest[BM];

  build_group_table(p, BM, s_ends, s_tile_pre, s_scan);
  const int total_tiles = s_tile_pre[p.e];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int64_t k = p.k, n = p.n;
  const int ktiles = (int)(k / BK);

  for (int t = blockIdx.x; t < total_tiles; t += gridDim.x) {
    const int g = find_group(s_tile_pre, p.e, t);
    const int local = t - s_tile_pre[g];
    const int mt = local / p.n_tiles_n, nt = local % p.n_tiles_n;
    const int64_t row_start = g ? s_ends[g - 1] : 0;
    const int64_t row_end = s_ends[g];
    const int64_t row0 = row_start + (int64_t)mt * BM;
    const int64_t col0 = (int64_t)nt * BN;

    // per-row epilogue factors for this tile
    for (int r = tid; r < BM; r += kThreads) {
      const int64_t row = row0 + r;
      const bool valid = row < row_end;
      s_pts[r] = (valid && p.pertoken) ? p.pertoken[row] : 1.0f;
      s_logit[r] = (valid && p.logit) ? p.logit[row] : 1.0f;
      s_dest[r] = valid ? (int32_t)dest_row(p, row) : -1;
    }

    // ---- global -> LDS copy of one k-stage
    const int8_t* x1 = p.x1;
    auto load_a = [&](int stage, int64_t k0) {
#pragma unroll
      for (int q = 0; q < (A_SLOTS + kThreads - 1) / kThreads; ++q) {
        const int slot_base = (q * NWAVES + wave) * 64;
        if (slot_base < A_SLOTS) {
          const int slot = slot_base + lane;
          const int r = slot / CPR_A, cpos = slot % CPR_A;
          const int c = cpos ^ swz_a<BK>(r);
          const int64_t row = min(row0 + r, p.m - 1);  // rows past the group: discarded later
          lds_dma16(x1 + row * k + k0 + c * 16, (LDS_PTR(void))(smA + stage * A_BYTES + slot_base * 16));
        }
      }
    };
    auto load_b8 = [&](int stage, int64_t k0) {
      const int8_t* w = (const int8_t*)p.x2 + (int64_t)g * k * n;
#pragma unroll
      for (int q = 0; q < (B_SLOTS + kThreads - 1) / kThreads; ++q) {
        const int slot_base = (q * NWAVES + wave) * 64;
        if (slot_base < B_SLOTS) {
          const int slot = slot_base + lane;
          const int r = slot / CPR_B, cpos = slot % CPR_B;
          const int c = cpos ^ swz_b(r);
          const int64_t col = min(col0 + c * 16, n - 16);  // columns past n: discarded later
          lds_dma16(w + (k0 + r) * n + col, (LDS_PTR(void))(smB + stage * B_BYTES + slot_base * 16));
        }
      }
    };
    // int4: each lane fetches 16 bytes = 32 packed columns, unpacks to two
    // 16-byte int8 chunks (values x16) and writes them to LDS itself.
    constexpr int B4_CHUNKS = BK * (BN / 32);
    constexpr int B4_PER_THREAD = (B4_CHUNKS + kThreads - 1) / kThreads;
    uint4 b4reg[INT4 ? B4_PER_THREAD : 1];
    auto fetch_b4 = [&](int64_t k0) {
      const uint32_t* w = (const uint32_t*)p.x2 + (int64_t)g * k * (n / 8);
#pragma unroll
      for (int q = 0; q < B4_PER_THREAD; ++q) {
        const int s = q * kThreads + tid;
        if (s < B4_CHUNKS) {
          const int r = s / (BN / 32), cc = s % (BN / 32);
          const int64_t col = min(col0 + cc * 32, n - 32);
          b4reg[q] = *(const uint4*)(w + (k0 + r) * (n / 8) + col / 8);
        }
      }
    };
    auto store_b4 = [&](int stage) {
#pragma unroll
      for (int q = 0; q < B4_PER_THREAD; ++q) {
        const int s = q * kThreads + tid;
        if (s < B4_CHUNKS) {
          const int r = s / (BN / 32), cc = s % (BN / 32);
          uint4 c0, c1;
          unpack_int4_x16(b4reg[q].x, c0.x, c0.y);
          unpack_int4_x16(b4reg[q].y, c0.z, c0.w);
          unpack_int4_x16(b4reg[q].z, c1.x, c1.y);
          unpack_int4_x16(b4reg[q].w, c1.z, c1.w);
          int8_t* base = smB + stage * B_BYTES + r * BN;
          *(uint4*)(base + (((2 * cc) ^ swz_b(r)) << 4)) = c0;
          *(uint4*)(base + (((2 * cc + 1) ^ swz_b(r)) << 4)) = c1;
        }
      }
    };

    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v16i{0};

    // prologue: stage 0
    load_a(0, 0);
    if constexpr (INT4) {
      fetch_b4(0);
      store_b4(0);
    } else {
      load_b8(0, 0);
    }

    for (int kt = 0; kt < ktiles; ++kt) {
      const int cur = kt & 1;
      __syncthreads();  // stage `cur` landed; everyone is done with stage cur^1
      const bool more = kt + 1 < ktiles;
      if (more) {
        load_a(cur ^ 1, (int64_t)(kt + 1) * BK);
        if constexpr (INT4) fetch_b4((int64_t)(kt + 1) * BK);
        else load_b8(cur ^ 1, (int64_t)(kt + 1) * BK);
      }
      const int8_t* As = smA + cur * A_BYTES;
      const int8_t* Bs = smB + cur * B_BYTES;
#pragma unroll
      for (int kk = 0; kk < BK / 32; ++kk) {
        v4i af[FM], bf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * WTM + i * 32 + (lane & 31);
          const int c = kk * 2 + (lane >> 5);
          af[i] = *(const LDS_PTR(v4i))(As + r * BK + ((c ^ swz_a<BK>(r)) << 4));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = kk * 32 + (lane >> 5) * 16 + ((lane & 15) >> 1);
          const int col = wn * WTN + j * 32 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
          const int8_t* a0 = Bs + r * BN + (((col >> 4) ^ swz_b(r)) << 4) + (col & 15);
          // rows r and r+8 share the same swizzle (r & 7)
          const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(v2i))(a0));
          const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(v2i))(a0 + 8 * BN));
          bf[j] = v4i{lo.x, lo.y, hi.x, hi.y};
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
      if constexpr (INT4) {
        if (more) store_b4(cur ^ 1);
      }
    }

    // ---- epilogue: lane holds rows (r/4)*8 + (lane/32)*4 + r%4, column lane%32
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int lc = wn * WTN + j * 32 + (lane & 31);
      const int64_t col = col0 + lc;
      const bool col_ok = col < n;
      float s = 1.0f;
      if (p.scale && col_ok)
        s = p.scale_bf16 ? bf16_to_f32(((const uint16_t*)p.scale)[(int64_t)g * n + col])
                         : ((const float*)p.scale)[(int64_t)g * n + col];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = wm * WTM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int64_t row = row0 + lr;
          if (!col_ok || row >= row_end) continue;
          int32_t a = acc[i][j][r];
          if constexpr (INT4) a >>= 4;  // weights were staged as 16 * w
          if (p.acc_out) p.acc_out[row * n + col] = a;
          float v = (float)a;           // v_cvt_f32_i32: round to nearest even
          v = v * s;
          v = v * s_pts[lr];
          v = v * s_logit[lr];
          if (p.combine == kCombineOrdered) {
            p.y[row * n + col] = v;
          } else {
            const int32_t d = s_dest[lr];
            if (d >= 0) __hip_atomic_fetch_add(p.out + (int64_t)d * n + col, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    __syncthreads();  // s_pts / s_logit / s_dest and LDS stages are reused by the next tile
  }
}

// ---------------------------------------------------------------------------
// out := seed.  Rows [off, off+bsdp) take the widened bf16 sharedInput, the
// rest +0.0 ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", Atlas 350 common
// constraints on sharedInput / sharedInputOffset / outputBS).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float4 seed4(const KParams& p, int64_t d, int64_t j4) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (p.shared && d >= p.shared_offset && d < p.shared_offset + p.bsdp) {
    const uint2 raw = *(const uint2*)(p.shared + (d - p.shared_offset) * p.n + j4 * 4);
    v.x = __uint_as_float(raw.x << 16);
    v.y = __uint_as_float(raw.x & 0xFFFF0000u);
    v.z = __uint_as_float(raw.y << 16);
    v.w = __uint_as_float(raw.y & 0xFFFF0000u);
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void seed_kernel(KParams p) {
  const int64_t n4 = p.n / 4, total = p.output_bs * n4;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * kThreads) {
    const int64_t d = idx / n4, j4 = idx % n4;
    *(float4*)(p.out + d * p.n + j4 * 4) = seed4(p, d, j4);
  }
}

// ---------------------------------------------------------------------------
// Ordered combine: bucket rows by destination, then fold each destination's
// rows in ascending source order onto the seed.  The order of additions is a
// function of the inputs only, so the result is bit-reproducible.
// ---------------------------------------------------------------------------

// Rows covered by the groups, clamped as in build_group_table (block-wide).
__device__ int64_t block_covered_rows(const KParams& p, int64_t* s_red) {
  const int tid = threadIdx.x;
  int64_t acc = 0;
  for (int g = tid; g < p.e; g += kThreads) {
    const int64_t x = min(max(p.group_list[g], (int64_t)0), p.m);
    acc = p.group_list_type == 0 ? max(acc, x) : acc + x;
  }
  s_red[tid] = acc;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) s_red[tid] = p.group_list_type == 0 ? max(s_red[tid], s_red[tid + off]) : s_red[tid] + s_red[tid + off];
    __syncthreads();
  }
  const int64_t c = min(s_red[0], p.m);
  __syncthreads();
  return c;
}

__global__ __launch_bounds__(kThreads) void fill_i32_kernel(int32_t* ptr, int64_t count, int32_t value) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += (int64_t)gridDim.x * kThreads) ptr[i] = value;
}

__global__ __launch_bounds__(kThreads) void hist_kernel(KParams p, int32_t* counts) {
  __shared__ int64_t s_red[kThreads];
  const int64_t covered = block_covered_rows(p, s_red);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < covered; i += (int64_t)gridDim.x * kThreads) {
    const int64_t d = dest_row(p, i);
    if (d >= 0) atomicAdd(counts + d, 1);
  }
}

// Single workgroup of 1024 threads: exclusive scan of counts into offsets
// (output_bs + 1 entries) and cursor := offsets.
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* counts, int32_t* offsets, int32_t* cursor, int64_t nbins) {
  __shared__ int32_t s[1024];
  const int tid = threadIdx.x;
  const int64_t per = (nbins + 1023) / 1024;
  const int64_t b0 = tid * per, b1 = min(b0 + per, nbins);
  int32_t local = 0;
  for (int64_t b = b0; b < b1; ++b) local += counts[b];
  s[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t t = tid >= off ? s[tid - off] : 0;
    __syncthreads();
    s[tid] += t;
    __syncthreads();
  }
  int32_t run = tid > 0 ? s[tid - 1] : 0;
  for (int64_t b = b0; b < b1; ++b) {
    offsets[b] = run;
    cursor[b] = run;
    run += counts[b];
  }
  if (tid == 1023) offsets[nbins] = s[1023];
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(KParams p, int32_t* cursor, int32_t* list) {
  __shared__ int64_t s_red[kThreads];
  const int64_t covered = block_covered_rows(p, s_red);
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < covered; i += (int64_t)gridDim.x * kThreads) {
    const int64_t d = dest_row(p, i);
    if (d >= 0) list[atomicAdd(cursor + d, 1)] = (int32_t)i;
  }
}

constexpr int kSegMax = 1024;  // longer segments take the scanning path

// One workgroup per destination row (grid-stride).  The destination's rows
// (unordered after the scatter) are ranked in LDS -- ranks are unique because
// row ids are -- then every column folds seed + y[rows] in ascending order.
__global__ __launch_bounds__(kThreads) void reduce_kernel(KParams p, const int32_t* offsets, const int32_t* list) {
  __shared__ int32_t s_src[kSegMax];
  __shared__ int32_t s_sorted[kSegMax];
  __shared__ int32_t s_dst[kThreads];
  __shared__ int64_t s_red[kThreads];
  const int tid = threadIdx.x;
  const int64_t n = p.n, n4 = n / 4;
  int64_t covered = -1;
  for (int64_t d = blockIdx.x; d < p.output_bs; d += gridDim.x) {
    const int32_t beg = offsets[d];
    const int32_t len = offsets[d + 1] - beg;
    if (len <= kSegMax) {
      for (int i = tid; i < len; i += kThreads) s_src[i] = list[beg + i];
      __syncthreads();
      for (int i = tid; i < len; i += kThreads) {
        const int32_t x = s_src[i];
        int rank = 0;
        for (int j = 0; j < len; ++j) rank += s_src[j] < x;
        s_sorted[rank] = x;
      }
      __syncthreads();
      for (int64_t j4 = tid; j4 < n4; j4 += kThreads) {
        float4 v = seed4(p, d, j4);
        for (int s = 0; s < len; ++s) {
          const float4 y = *(const float4*)(p.y + (int64_t)s_sorted[s] * n + j4 * 4);
          v.x = v.x + y.x;
          v.y = v.y + y.y;
          v.z = v.z + y.z;
          v.w = v.w + y.w;
        }
        *(float4*)(p.out + d * n + j4 * 4) = v;
      }
      __syncthreads();
    } else {
      // Long segment: walk all covered rows in ascending order.
      if (covered < 0) covered = block_covered_rows(p, s_red);
      for (int64_t j4b = 0; j4b < n4; j4b += kThreads) {
        const int64_t j4 = j4b + tid;
        float4 v = j4 < n4 ? seed4(p, d, j4) : make_float4(0.f, 0.f, 0.f, 0.f);
        for (int64_t i0 = 0; i0 < covered; i0 += kThreads) {
          const int64_t i = i0 + tid;
          s_dst[tid] = i < covered ? (int32_t)dest_row(p, i) : -1;
          __syncthreads();
          const int cnt = (int)min((int64_t)kThreads, covered - i0);
          if (j4 < n4) {
            for (int c = 0; c < cnt; ++c) {
              if (s_dst[c] != d) continue;
              const float4 y = *(const float4*)(p.y + (i0 + c) * n + j4 * 4);
              v.x = v.x + y.x;
              v.y = v.y + y.y;
              v.z = v.z + y.z;
              v.w = v.w + y.w;
            }
          }
          __syncthreads();
        }
        if (j4 < n4) *(float4*)(p.out + d * n + j4 * 4) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
TileShape tile_shape(TileId id) {
  switch (id) {
    case kTile256x256: return {256, 256, 64};
    case kTile128x256: return {128, 256, 64};
    case kTile64x256: return {64, 256, 64};
    default: return {32, 256, 64};
  }
}

int tile_occupancy(TileId id) { return id == kTile256x256 ? 1 : 2; }

const char* tile_kernel_name(TileId id, bool int4) {
  static const char* names[kNumTiles][2] = {
      {"gmm_kernel<256,256,64,2x2,i8>", "gmm_kernel<256,256,64,2x2,i4>"},
      {"gmm_kernel<128,256,64,2x2,i8>", "gmm_kernel<128,256,64,2x2,i4>"},
      {"gmm_kernel<64,256,64,1x4,i8>", "gmm_kernel<64,256,64,1x4,i4>"},
      {"gmm_kernel<32,256,64,1x4,i8>", "gmm_kernel<32,256,64,1x4,i4>"},
  };
  return names[(int)id][int4 ? 1 : 0];
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

OrderedWorkspace ordered_workspace(int64_t m, int64_t n, int64_t output_bs) {
  OrderedWorkspace w;
  size_t off = 0;
  w.y_off = off;
  off += align256((size_t)m * (size_t)n * sizeof(float));
  w.counts_off = off;
  off += align256((size_t)output_bs * 4);
  w.cursor_off = off;
  off += align256((size_t)output_bs * 4);
  w.offsets_off = off;
  off += align256((size_t)(output_bs + 1) * 4);
  w.list_off = off;
  off += align256((size_t)(m > 0 ? m : 1) * 4);
  w.total = off;
  return w;
}

template <int BM, int BN, int BK, int WM, int WN, int OCC>
static void launch_gemm(const KParams& kp, bool int4, int grid, hipStream_t s) {
  if (int4) hipLaunchKernelGGL((gmm_kernel<BM, BN, BK, WM, WN, OCC, true>), dim3(grid), dim3(kThreads), 0, s, kp);
  else hipLaunchKernelGGL((gmm_kernel<BM, BN, BK, WM, WN, OCC, false>), dim3(grid), dim3(kThreads), 0, s, kp);
}

int launch_all(const LaunchArgs& a, const Plan& plan, void* workspace, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const TileShape ts = tile_shape(plan.tile);
  KParams kp;
  kp.x1 = a.x1;
  kp.x2 = a.x2;
  kp.scale = a.scale;
  kp.pertoken = a.pertoken;
  kp.logit = a.logit;
  kp.group_list = a.group_list;
  kp.row_index = a.row_index;
  kp.shared = a.shared;
  kp.out = a.out;
  kp.y = nullptr;
  kp.acc_out = a.acc_out;
  kp.m = a.m;
  kp.k = a.k;
  kp.n = a.n;
  kp.bsdp = a.bsdp;
  kp.shared_offset = a.shared_offset;
  kp.output_bs = a.output_bs;
  kp.e = a.e;
  kp.group_list_type = a.group_list_type;
  kp.scale_bf16 = a.scale_bf16;
  kp.row_index_i32 = a.row_index_i32;
  kp.n_tiles_n = (int32_t)((a.n + ts.bn - 1) / ts.bn);
  kp.combine = plan.combine;

  const int64_t n4 = a.n / 4;
  if (plan.combine == kCombineOrdered) {
    const OrderedWorkspace w = ordered_workspace(a.m, a.n, a.output_bs);
    char* ws = (char*)workspace;
    kp.y = (float*)(ws + w.y_off);
    int32_t* counts = (int32_t*)(ws + w.counts_off);
    int32_t* cursor = (int32_t*)(ws + w.cursor_off);
    int32_t* offsets = (int32_t*)(ws + w.offsets_off);
    int32_t* list = (int32_t*)(ws + w.list_off);
    const int gb = (int)std::min<int64_t>(1024, (a.output_bs + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(gb), dim3(kThreads), 0, s, counts, a.output_bs, 0);
    if (a.m > 0) {
      const int gm = (int)std::min<int64_t>(2048, (a.m + kThreads - 1) / kThreads);
      hipLaunchKernelGGL(hist_kernel, dim3(gm), dim3(kThreads), 0, s, kp, counts);
      hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, counts, offsets, cursor, a.output_bs);
      hipLaunchKernelGGL(scatter_kernel, dim3(gm), dim3(kThreads), 0, s, kp, cursor, list);
    } else {
      hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, counts, offsets, cursor, a.output_bs);
    }
  } else {
    const int gs = (int)std::min<int64_t>(4096, (a.output_bs * n4 + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(seed_kernel, dim3(gs > 0 ? gs : 1), dim3(kThreads), 0, s, kp);
  }
  if (a.m > 0 && plan.grid > 0) {
    switch (plan.tile) {
      case kTile256x256: launch_gemm<256, 256, 64, 2, 2, 1>(kp, a.int4, plan.grid, s); break;
      case kTile128x256: launch_gemm<128, 256, 64, 2, 2, 2>(kp, a.int4, plan.grid, s); break;
      case kTile64x256: launch_gemm<64, 256, 64, 1, 4, 2>(kp, a.int4, plan.grid, s); break;
      default: launch_gemm<32, 256, 64, 1, 4, 2>(kp, a.int4, plan.grid, s); break;
    }
  }
  if (plan.combine == kCombineOrdered) {
    const OrderedWorkspace w = ordered_workspace(a.m, a.n, a.output_bs);
    char* ws = (char*)workspace;
    const int gr = (int)std::min<int64_t>(65535, a.output_bs);
    hipLaunchKernelGGL(reduce_kernel, dim3(gr > 0 ? gr : 1), dim3(kThreads), 0, s, kp,
                       (const int32_t*)(ws + w.offsets_off), (const int32_t*)(ws + w.list_off));
  }
  return (int)hipGetLastError();
}

}  // namespace gmmfr
