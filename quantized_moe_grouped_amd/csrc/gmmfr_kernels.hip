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
//   gmm_kernel<...>    persistent grouped int8 / int4 GEMM (256x256 tiles with
//                      eight waves, or 128/64/32 x 256 with four); epilogue adds
//                      into out with fp32 atomics, or stores y for the ordered
//                      combine
//   mx_gemm_kernel<..> the same for FP8 x FP4 (MxA8W4, E8M0 block scales) and
//                      FP8 x FP8 weights, on the block-scaled MFMA
//   hist/scan/scatter  rows bucketed by destination (ordered combine)
//   reduce_kernel      per destination: sort its rows ascending, fold
//                      seed + y[rows] in that order, write out once
//   reduce_scan_kernel the same without the buckets: each destination scans
//                      rowIndex for its rows (small m * outputBS)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

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
  int32_t pertoken_scalar;  // pertoken holds one value for every row
  int32_t n_tiles_n;
  int32_t combine;
  int32_t* tile_ctr;    // per-XCD tile queues (kTileQueues counters, 64 bytes apart), zeroed before the GEMM
  int32_t reduce_split; // ordered combine: workgroups (column ranges) per destination row, >= 1
  int32_t hyb_atomic;   // hybrid combine: atomic column tiles in each kHybridPeriod (0: not hybrid)
  int64_t n4_ord;       // float4 columns the ordered reduce folds (n / 4 unless hybrid)
  int64_t n4_seed;      // float4 columns the seed kernel writes (n / 4 unless hybrid)
  int32_t y_cached;     // the scan-lookup reduce with a small y: the GEMM stores y through the
                        // caches (two workgroups per CU only) and the reduce reads it so, from the
                        // MALL; otherwise both nontemporal
};

// Hybrid combine: float4 column of the jj-th float4 column of one class
// (the atomic column tiles, or the ordered ones) in ascending order.  A
// 256-column tile holds 64 float4 columns; tile nt is atomic when
// nt % kHybridPeriod < hyb_atomic.  The identity when not hybrid.
__device__ __forceinline__ int64_t hyb_col4(const KParams& p, int64_t jj, bool atomic_class) {
  if (p.hyb_atomic == 0) return jj;
  const int64_t per = atomic_class ? p.hyb_atomic : kHybridPeriod - p.hyb_atomic;
  const int64_t b = jj >> 6;
  return ((b / per) * kHybridPeriod + (atomic_class ? 0 : p.hyb_atomic) + b % per) * 64 + (jj & 63);
}

constexpr int64_t kYCachedBytes = int64_t(160) << 20;  // y small enough to wait in the MALL
constexpr int kTileQueues = 8;       // one per XCD
constexpr int kTileQueueStride = 16; // int32 elements between counters (one 64-byte line each)
constexpr int kTileBlock = 64;       // consecutive raster tiles handed to one XCD at a time

// XCD (XCC) the calling wave runs on.
__device__ __forceinline__ int xcc_id() {
  return (int)(__builtin_amdgcn_s_getreg((20) | (0 << 6) | ((16 - 1) << 11)) & (kTileQueues - 1));
}

// Tile of the j-th grab from queue q: raster blocks of kTileBlock tiles are
// dealt to the queues in turn.  -1 once past the last tile.
__device__ __forceinline__ int queue_tile(int q, int j, int total) {
  const int64_t t = ((int64_t)(j / kTileBlock) * kTileQueues + q) * kTileBlock + (j % kTileBlock);
  return t < total ? (int)t : -1;
}

// One grab from queue q, then from the other queues in turn until a tile is
// found or all are exhausted (-1).  Stealing only happens at the very end, and
// makes every tile processed whatever the placement of workgroups on XCDs.
__device__ __forceinline__ int grab_tile_from(int* ctr, int q, int total) {
  for (int tries = 0; tries < kTileQueues; ++tries) {
    const int qq = (q + tries) % kTileQueues;
    const int t = queue_tile(qq, atomicAdd(ctr + qq * kTileQueueStride, 1), total);
    if (t >= 0) return t;
  }
  return -1;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// A 64-bit value that is the same in every lane, moved to scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  return (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(x >> 32)) << 32) |
                   (uint32_t)__builtin_amdgcn_readfirstlane((int)x));
}

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
template <int NT>
__device__ void block_scan_i64(int64_t (&v)[kMaxExperts / NT], bool use_max, int64_t* s_scan) {
  constexpr int PER = kMaxExperts / NT;
  const int tid = threadIdx.x;
#pragma unroll
  for (int q = 1; q < PER; ++q) v[q] = use_max ? max(v[q - 1], v[q]) : v[q - 1] + v[q];
  s_scan[tid] = v[PER - 1];
  __syncthreads();
  for (int off = 1; off < NT; off <<= 1) {
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
template <int NT = kThreads>
__device__ void build_group_table(const KParams& p, int bm, int32_t* s_ends, int32_t* s_tile_pre, int64_t* s_scan) {
  constexpr int PER = kMaxExperts / NT;
  const int tid = threadIdx.x;
  int64_t v[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int g = tid * PER + q;
    int64_t x = g < p.e ? p.group_list[g] : 0;
    v[q] = min(max(x, (int64_t)0), p.m);
  }
  block_scan_i64<NT>(v, p.group_list_type == 0, s_scan);
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
  block_scan_i64<NT>(v, false, s_scan);
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
//            of k-row r is stored at position c ^ (2 * (r & 7)).  Read with
//            the gfx950 transpose load ds_read_b64_tr_b8: within each 16-lane
//            group, lane 16G+i receives byte (i % 8) of the eight 8-byte rows
//            addressed by lanes 16G + 2b + i/8 (b = 0..7).  Lane s therefore
//            supplies k-row (s%16)/2 at column 16*((s/16)%2) + 8*(s%2) and
//            gets eight consecutive k of column s%32; two such loads give the
//            16 k-values the i8 MFMA expects per lane.  The 32 lanes of one
//            pass touch 8 k-rows x 2 adjacent chunks; the even swizzle sends
//            them to 16 distinct chunk positions (all 64 banks), where r & 7
//            alone would fold the pair onto 8 positions (2-way conflicts).
// Both stages are filled by global_load_lds_dwordx4 (HBM -> LDS without
// VGPRs); a lane's LDS slot is fixed, so the swizzle is applied by choosing
// which global chunk each lane fetches.
// ---------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ int swz_a(int r) {
  if constexpr (BK == 64) return ((r >> 1) ^ (r >> 3)) & 3;
  else return (r ^ (r >> 3)) & 7;
}
__device__ __forceinline__ int swz_b(int r) { return (r & 7) << 1; }
// FP4 (MxA8W4) B stage: column r's two 16-byte chunks, swapped when bit 3 of r is set
__device__ __forceinline__ int swz_b4(int r) { return (r >> 3) & 1; }

// HBM -> LDS copy of 16 bytes per lane: lane i of the wave writes LDS bytes
// [lds_base + 16 i, lds_base + 16 i + 16).  lds_base must be wave-uniform.
// Written as inline asm so that the compiler does not track these LDS writes
// (it would otherwise wait for every copy in flight before each LDS read and
// each barrier); completion is awaited explicitly with wait_vmcnt before the
// workgroup barrier that publishes a stage.  M0 is set here and used by
// nothing else in these kernels.
__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gsrc) : "memory");
}
// Same copy with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane
// byte offset (saddr form): one VGPR per copy instead of two.
__device__ __forceinline__ void lds_dma16_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
               : "memory");
}

// 4 bytes per lane (global_load_lds_dword), saddr form: lane i writes LDS
// bytes [lds_base + 4 i, lds_base + 4 i + 4).  Inactive lanes write nothing.
__device__ __forceinline__ void lds_dma4_sv(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const LDS_PTR(void))p;
}

// Workgroup barrier that publishes LDS written by ds_write (lgkmcnt) but does
// not wait for copies in flight (the caller waits for those it needs).
__device__ __forceinline__ void lds_barrier() {
  // the compiler's own waitcnt tracking sees this lgkmcnt(0); the empty asm
  // statements keep memory accesses from moving across the barrier
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// One accumulator element read where it is used.  With accumulators in AGPRs
// this keeps the compiler from copying the whole accumulator array to VGPRs
// at once after the mainloop (which would need every VGPR and spill).
template <bool FROM_AGPR>
__device__ __forceinline__ int32_t acc_elem(int32_t x) {
  if constexpr (FROM_AGPR) {
    int32_t v;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(x));
    return v;
  } else {
    return x;
  }
}

// int4 word -> 8 int8 holding 16 * value, in column order (two dwords).
__device__ __forceinline__ void unpack_int4_x16(uint32_t w, uint32_t& d0, uint32_t& d1) {
  const uint32_t lo = (w << 4) & 0xF0F0F0F0u;  // 16*t0, 16*t2, 16*t4, 16*t6
  const uint32_t hi = w & 0xF0F0F0F0u;         // 16*t1, 16*t3, 16*t5, 16*t7
  d0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);  // t0 t1 t2 t3
  d1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // t4 t5 t6 t7
}

// Compile-time loop helper.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Tile order inside one expert: groups of group_m m-tiles, n-tiles swept
// inside a group with the m-tile fastest, so the tiles resident on one XCD
// at a time (64 of 128 rows: 8 m x 8 n; 32 of 256 rows: 4 m x 8 n) share A
// row panels and B column panels in that XCD's L2.  For the 256-row tile,
// groups of 4 measured 0.7-1.4% faster than groups of 8 (and 2 alike, 16
// 7% slower); for 128-row tiles groups of 8 beat 4 by 1.6%.
template <int BM>
constexpr int group_m() { return BM >= 256 ? 4 : 8; }

// Position of one output tile.
struct TileCoord {
  int g;            // expert
  int64_t row0;     // first row of the tile in x1
  int64_t col0;     // first column
  int valid_rows;   // rows of the tile inside the expert's group (<= BM)
};

template <int BM, int BN>
__device__ __forceinline__ TileCoord tile_coord(const KParams& p, const int32_t* s_ends, const int32_t* s_tile_pre,
                                                int t) {
  TileCoord c;
  c.g = find_group(s_tile_pre, p.e, t);
  const int local = t - s_tile_pre[c.g];
  const int64_t row_start = c.g ? s_ends[c.g - 1] : 0;
  const int64_t row_end = s_ends[c.g];
  const int mtiles = (int)((row_end - row_start + BM - 1) / BM);
  constexpr int GM = group_m<BM>();
  const int grp = local / (GM * p.n_tiles_n);
  const int in_grp = local - grp * GM * p.n_tiles_n;
  const int gsize = min(GM, mtiles - grp * GM);
  const int mt = grp * GM + in_grp % gsize;
  const int nt = in_grp / gsize;
  c.row0 = row_start + (int64_t)mt * BM;
  c.col0 = (int64_t)nt * BN;
  c.valid_rows = (int)min((int64_t)BM, row_end - c.row0);
  return c;
}

// CONT selects the continuous copy pipeline (int8 weights, k / BK >= STAGES,
// checked by the host) over the tile-by-tile loop.  TRANSB: int8 weights
// given transposed, (e,n,k) with k contiguous.
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int OCC, bool INT4, int COMBINE, bool CONT,
          bool TRANSB, int NT = kThreads>
__global__ __launch_bounds__(NT, OCC) void gmm_kernel(KParams p) {
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int KK = BK / 32;
  // int4 weights in the continuous pipeline stay packed in LDS (two columns
  // per byte); the tile-by-tile loop unpacks them on the way in.
  constexpr bool PACKED = INT4 && CONT;
  constexpr bool REGB4 = INT4 && !CONT;  // int4 B through registers
  // Transposed int8 weights: a B stage is laid out like an A stage, one LDS
  // row of BK bytes per weight column, and read like it.
  constexpr bool TB = TRANSB;
  static_assert(!(TRANSB && INT4), "transposed weights are int8");
  constexpr int B_ROW = TB ? BK : (PACKED ? BN / 2 : BN);  // bytes of one LDS row of a B stage
  constexpr int B_LROWS = TB ? BN : BK;                    // LDS rows of a B stage
  constexpr int CPR_A = BK / 16, CPR_B = B_ROW / 16;
  constexpr int A_BYTES = BM * BK, B_BYTES = B_LROWS * B_ROW;
  constexpr int A_SLOTS = BM * CPR_A, B_SLOTS = B_LROWS * CPR_B;
  constexpr int NWAVES = NT / 64;
  constexpr int A_INSTR = (A_SLOTS + NT - 1) / NT;    // per thread (whole waves may idle)
  constexpr int B_INSTR = (B_SLOTS + NT - 1) / NT;
  constexpr int B4_CHUNKS = BK * (BN / 32);                       // 16-byte packed chunks
  constexpr int B4_PER = (B4_CHUNKS + NT - 1) / NT;
  // vector-memory ops one thread issues per stage (DMA and int4 register
  // loads).  When A_SLOTS is not a multiple of the block, the last A copy is
  // issued by the first waves only; those waves wait with the larger count.
  constexpr int B_ISSUED = REGB4 ? B4_PER : B_INSTR;
  constexpr int LOADS_FULL = A_INSTR + B_ISSUED;
  constexpr int LOADS_SHORT = A_INSTR - 1 + B_ISSUED;
  static_assert(WAVES_M * WAVES_N == NWAVES, "waves cover the workgroup");
  static_assert(FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0, "wave tile");
  static_assert(BN >= 256, "B swizzle needs 16 chunks per row (8 when packed)");
  static_assert(A_SLOTS % 64 == 0 && B_SLOTS % 64 == 0, "whole waves per copy");
  static_assert(STAGES >= 2 && STAGES <= 4, "stages");
  static_assert((STAGES - 2) * LOADS_FULL < 64, "vmcnt range");
  static_assert(KK % 2 == 0, "fragment double buffer alternates within a stage");

  __shared__ __attribute__((aligned(16))) int8_t sA[STAGES * A_BYTES];
  __shared__ __attribute__((aligned(16))) int8_t sB[STAGES * B_BYTES];
  // per-expert tables, sized by e at launch: ends[e], tile prefix[e + 1]
  extern __shared__ __attribute__((aligned(16))) int32_t s_dyn[];
  int32_t* s_ends = s_dyn;
  int32_t* s_tile_pre = s_dyn + p.e;
  int64_t* s_scan = (int64_t*)sA;  // scan scratch, used before the first copy into sA
  static_assert(STAGES * A_BYTES >= NT * 8, "scan scratch fits in the A stages");
  // Per-row epilogue inputs of a tile (pertokenScale, logit, rowIndex) and
  // per-column scales, as raw words of the caller's arrays, double-buffered
  // across consecutive tiles: rowIndex takes two words per row when int64,
  // one when int32; the scale one word per column (fp32) or per column pair
  // (bf16).
  __shared__ __attribute__((aligned(16))) float s_pts[2][BM];
  __shared__ __attribute__((aligned(16))) float s_logit[2][BM];
  __shared__ __attribute__((aligned(16))) uint32_t s_ridx[2][2 * BM];
  __shared__ __attribute__((aligned(16))) uint32_t s_scale[2][BN];

  // An absent pertokenScale or logit reads as 1.0 from LDS (the copies below
  // skip it), so the epilogue reads row factors without branching; a
  // per-tensor pertokenScale is filled in once the same way.  The barriers
  // of the table build publish the fill.
  const bool pts_rows = p.pertoken && !p.pertoken_scalar;
  if (!pts_rows) {
    const float v = p.pertoken ? p.pertoken[0] : 1.0f;
    for (int i = threadIdx.x; i < 2 * BM; i += NT) (&s_pts[0][0])[i] = v;
  }
  if (!p.logit)
    for (int i = threadIdx.x; i < 2 * BM; i += NT) (&s_logit[0][0])[i] = 1.0f;
  build_group_table<NT>(p, BM, s_ends, s_tile_pre, s_scan);
  const int total_tiles = s_tile_pre[p.e];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lane_id = lane, wave_m = wm, wave_n = wn;
  // B chunk swizzle.  Packed rows hold 8 chunks: a 32-lane pass of the
  // transpose read covers 8 k-rows x 2 adjacent chunks, two rows per bank
  // cycle; 2((r >> 1) & 3) sends the rows of one parity to 8 distinct chunk
  // positions.
  auto swzb = [](int r) { return PACKED ? ((r >> 1) & 3) << 1 : swz_b(r); };
  const bool a_full = ((A_INSTR - 1) * NWAVES + wave) * 64 < A_SLOTS;  // wave-uniform
  const int64_t k = p.k, n = p.n;
  const int ktiles = (int)(k / BK);

  __shared__ int s_tiles[2];
  const int xcd = xcc_id();
  // Tile coordinates are the same for every lane; say so, so that they stay
  // in scalar registers.
  auto coord = [&](int tt) {
    TileCoord c = tile_coord<BM, BN>(p, s_ends, s_tile_pre, __builtin_amdgcn_readfirstlane(tt));
    c.g = __builtin_amdgcn_readfirstlane(c.g);
    c.valid_rows = __builtin_amdgcn_readfirstlane(c.valid_rows);
    c.row0 = uniform64(c.row0);
    c.col0 = uniform64(c.col0);
    return c;
  };

  // ---- per-tile copy sources: wave-uniform bases plus per-lane offsets
  // (bytes, < BM*k resp. < BK*n, so they fit in 32 bits)
  uint32_t a_off[A_INSTR];
  uint32_t b_off[REGB4 ? 1 : B_INSTR];
  const int8_t* a_base = p.x1;
  const int8_t* b_base = nullptr;
  const uint32_t* w4 = nullptr;
  int64_t b4_col0 = 0;
  uint4 b4reg[REGB4 ? B4_PER : 1];
  auto set_sources = [&](const TileCoord& c) {
    // copy bases are wave-uniform (SGPRs: the copies' saddr operand)
    a_base = (const int8_t*)uniform64((int64_t)(p.x1 + c.row0 * k));
#pragma unroll
    for (int q = 0; q < A_INSTR; ++q) {
      const int slot = (q * NWAVES + wave) * 64 + lane;
      const int r = (slot / CPR_A) % BM, cpos = slot % CPR_A;
      const int64_t row = min(c.row0 + r, p.m - 1);  // rows past the group: loaded, never stored
      a_off[q] = (uint32_t)((row - c.row0) * k + ((cpos ^ swz_a<BK>(r)) * 16));
    }
    if constexpr (TB) {
      // weight column col is k contiguous bytes; columns past n: loaded, never stored
      b_base = (const int8_t*)uniform64((int64_t)((const int8_t*)p.x2 + ((int64_t)c.g * n + c.col0) * k));
#pragma unroll
      for (int q = 0; q < B_INSTR; ++q) {
        const int slot = (q * NWAVES + wave) * 64 + lane;
        const int r = (slot / CPR_B) % BN, cpos = slot % CPR_B;
        const int64_t col = min(c.col0 + r, n - 1);
        b_off[q] = (uint32_t)((col - c.col0) * k + ((cpos ^ swz_a<BK>(r)) * 16));
      }
    } else if constexpr (!REGB4) {
      // bytes of one weight row, and the tile's first byte in it
      const int64_t rowb = PACKED ? n / 2 : n, col0b = PACKED ? c.col0 / 2 : c.col0;
      b_base = (const int8_t*)uniform64((int64_t)((const int8_t*)p.x2 + (int64_t)c.g * k * rowb + col0b));
#pragma unroll
      for (int q = 0; q < B_INSTR; ++q) {
        const int slot = (q * NWAVES + wave) * 64 + lane;
        const int r = (slot / CPR_B) % BK, cpos = slot % CPR_B;
        const int64_t colb = min(col0b + ((cpos ^ swzb(r)) * 16), rowb - 16);  // past n: loaded, never stored
        b_off[q] = (uint32_t)((int64_t)r * rowb + (colb - col0b));
      }
    } else {
      w4 = (const uint32_t*)p.x2 + (int64_t)c.g * k * (n / 8);
      b4_col0 = c.col0;
    }
  };

  auto issue_a = [&](int sc, int kt) {
    const int8_t* base = a_base + (int64_t)kt * BK;
#pragma unroll
    for (int q = 0; q < A_INSTR; ++q) {
      const int slot_base = (q * NWAVES + wave) * 64;
      if ((A_SLOTS % (NWAVES * 64)) == 0 || slot_base < A_SLOTS)
        lds_dma16_sv(base, a_off[q], __builtin_amdgcn_readfirstlane(lds_addr(sA + sc * A_BYTES + slot_base * 16)));
    }
  };
  auto issue_b8 = [&](int sc, int kt) {
    const int8_t* base = b_base + (int64_t)kt * BK * (TB ? 1 : (PACKED ? n / 2 : n));
#pragma unroll
    for (int q = 0; q < B_INSTR; ++q) {
      const int slot_base = (q * NWAVES + wave) * 64;
      if ((B_SLOTS % (NWAVES * 64)) == 0 || slot_base < B_SLOTS)
        lds_dma16_sv(base, b_off[q], __builtin_amdgcn_readfirstlane(lds_addr(sB + sc * B_BYTES + slot_base * 16)));
    }
  };
  auto fetch_b4 = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
    for (int q = 0; q < B4_PER; ++q) {
      const int s = q * NT + tid;
      if (s < B4_CHUNKS) {
        const int r = s / (BN / 32), cc = s % (BN / 32);
        const int64_t col = min(b4_col0 + cc * 32, n - 32);
        b4reg[q] = *(const uint4*)(w4 + (k0 + r) * (n / 8) + col / 8);
      }
    }
  };
  auto store_b4 = [&](int sc) {
#pragma unroll
    for (int q = 0; q < B4_PER; ++q) {
      const int s = q * NT + tid;
      if (s < B4_CHUNKS) {
        const int r = s / (BN / 32), cc = s % (BN / 32);
        uint4 c0, c1;
        unpack_int4_x16(b4reg[q].x, c0.x, c0.y);
        unpack_int4_x16(b4reg[q].y, c0.z, c0.w);
        unpack_int4_x16(b4reg[q].z, c1.x, c1.y);
        unpack_int4_x16(b4reg[q].w, c1.z, c1.w);
        int8_t* base = sB + sc * B_BYTES + r * BN;
        *(uint4*)(base + (((2 * cc) ^ swz_b(r)) << 4)) = c0;
        *(uint4*)(base + (((2 * cc + 1) ^ swz_b(r)) << 4)) = c1;
      }
    }
  };
  // stage fill: int4 issues its register loads first so that waiting for
  // them later does not also wait for the A copy issued after them
  auto issue_stage = [&](int sc, int kt) {
    if constexpr (REGB4) {
      fetch_b4(kt);
      issue_a(sc, kt);
    } else {
      issue_a(sc, kt);
      issue_b8(sc, kt);
    }
  };
  // stages 0 .. STAGES-2 of a tile (the buffers must be free)
  auto prologue = [&]() {
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st) {
      if (st < ktiles) {
        issue_stage(st, st);
        if constexpr (REGB4) store_b4(st);
      }
    }
  };
  // Per-row and per-column epilogue inputs of a tile into buffer `pb`, as raw
  // words.  Rows past the group or past m and columns past n read a clamped,
  // valid address; the epilogue never uses them.
  // rowIndex words per tile: only the atomic combine reads them here
  const int ridx_words = (COMBINE != kCombineOrdered && p.row_index) ? (p.row_index_i32 ? BM : 2 * BM) : 0;
  const int scale_words = p.scale ? (p.scale_bf16 ? BN / 2 : BN) : 0;
  auto row_word_src = [&](const TileCoord& c, int q, int words_per_row) -> int64_t {
    const int64_t row = min(c.row0 + q / words_per_row, p.m - 1);
    return row * words_per_row + q % words_per_row;  // word index into the array
  };
  auto scale_word_src = [&](const TileCoord& c, int q) -> int64_t {
    // fp32: one column per word; bf16: columns 2q, 2q+1 (n is even)
    if (p.scale_bf16) return ((int64_t)c.g * n + min(c.col0 + 2 * q, n - 2)) / 2;
    return (int64_t)c.g * n + min(c.col0 + q, n - 1);
  };
  // Register path (the k-loop with a tile prologue): loads now, LDS writes later.
  // (an absent pertokenScale or logit stays 1.0)
  uint32_t fr_pts = 0x3F800000u, fr_logit = 0x3F800000u, fr_ridx0 = 0, fr_ridx1 = 0, fr_scale = 0;
  auto fetch_rows = [&](const TileCoord& c) {
    if (tid < BM) {
      if (pts_rows) fr_pts = ((const uint32_t*)p.pertoken)[row_word_src(c, tid, 1)];
      if (p.logit) fr_logit = ((const uint32_t*)p.logit)[row_word_src(c, tid, 1)];
    }
    const uint32_t* ri = (const uint32_t*)p.row_index;
    if (tid < ridx_words) fr_ridx0 = ri[row_word_src(c, tid, ridx_words / BM)];
    if (tid + NT < ridx_words) fr_ridx1 = ri[row_word_src(c, tid + NT, ridx_words / BM)];
    if (tid < scale_words) fr_scale = ((const uint32_t*)p.scale)[scale_word_src(c, tid)];
  };
  auto store_rows = [&](int pb) {
    if (tid < BM) {
      if (pts_rows) s_pts[pb][tid] = __uint_as_float(fr_pts);
      s_logit[pb][tid] = __uint_as_float(fr_logit);
    }
    if (tid < ridx_words) s_ridx[pb][tid] = fr_ridx0;
    if (tid + NT < ridx_words) s_ridx[pb][tid + NT] = fr_ridx1;
    if (tid < scale_words) s_scale[pb][tid] = fr_scale;
  };
  // Copy path (the continuous pipeline): straight to LDS, one word per lane,
  // from a per-tile base so that lane offsets stay small.  Issued before the
  // k-step copies that follow, so the stage waits cover them.
  auto dma_rows = [&](const TileCoord& c, int pb) {
    auto words = [&](const uint32_t* base_any, uint32_t* dst, int nwords, auto&& word_off) {
      const uint32_t* base = (const uint32_t*)uniform64((int64_t)base_any);  // the same in every lane
      const int q = wave * 64 + lane;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int qq = q + pass * NT;
        if (pass * NT + wave * 64 < nwords) {  // wave-uniform
          if (qq < nwords)
            lds_dma4_sv(base, (uint32_t)word_off(qq) * 4u,
                        __builtin_amdgcn_readfirstlane(lds_addr(dst + pass * NT + wave * 64)));
        }
      }
    };
    // Clamps in 32 bits against a wave-uniform limit (rows of the tile that
    // exist in x1, columns that exist in the weight): a 64-bit per-lane row
    // index here was spilled and reloaded behind a full memory wait per tile.
    const int row_lim = (int)min(p.m - 1 - c.row0, (int64_t)BM);
    const int col_lim = (int)min(n - 1 - c.col0, (int64_t)BN);
    auto row_off = [&](int q, int wpr) { return min(q / wpr, row_lim) * wpr + q % wpr; };
    if (pts_rows)
      words((const uint32_t*)p.pertoken + c.row0, (uint32_t*)s_pts[pb], BM, [&](int q) { return row_off(q, 1); });
    if (p.logit)
      words((const uint32_t*)p.logit + c.row0, (uint32_t*)s_logit[pb], BM, [&](int q) { return row_off(q, 1); });
    if (ridx_words) {
      const int wpr = ridx_words / BM;
      words((const uint32_t*)p.row_index + c.row0 * wpr, s_ridx[pb], ridx_words, [&](int q) { return row_off(q, wpr); });
    }
    if (scale_words) {
      if (p.scale_bf16)
        words((const uint32_t*)((const uint16_t*)p.scale + (int64_t)c.g * n + c.col0), s_scale[pb], scale_words,
              [&](int q) { return min(2 * q, col_lim - 1) / 2; });
      else
        words((const uint32_t*)p.scale + (int64_t)c.g * n + c.col0, s_scale[pb], scale_words,
              [&](int q) { return min(q, col_lim); });
    }
  };
  static_assert(BM <= NT && BN <= NT && 2 * BM <= 2 * NT, "one pass per tile row and column");

  // Fragment reads.  Read item r of a k-substep: A fragments first, then B.
  auto read_a = [&](int sc, int kk, int i, v4i& dst) {
    const int r = wm * WTM + i * 32 + (lane & 31);
    const int c = kk * 2 + (lane >> 5);
    dst = *(const LDS_PTR(v4i))(sA + sc * A_BYTES + r * BK + ((c ^ swz_a<BK>(r)) << 4));
  };
  auto read_b = [&](int sc, int kk, int j, v4i& dst) {
    if constexpr (TB) {
      // column-major stage: the same lane layout as the A fragment
      const int rc = wn * WTN + j * 32 + (lane & 31);
      const int cc = kk * 2 + (lane >> 5);
      dst = *(const LDS_PTR(v4i))(sB + sc * B_BYTES + rc * BK + ((cc ^ swz_a<BK>(rc)) << 4));
    } else {
      const int r = kk * 32 + (lane >> 5) * 16 + ((lane & 15) >> 1);
      const int col = wn * WTN + j * 32 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
      const int8_t* a0 = sB + sc * B_BYTES + r * B_ROW + (((col >> 4) ^ swzb(r)) << 4) + (col & 15);
      const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(v2i))(a0));
      const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(v2i))(a0 + 8 * B_ROW));  // same swizzle
      dst = v4i{lo.x, lo.y, hi.x, hi.y};
    }
  };
  // Packed int4: one transpose read of byte column b gives, per k, the
  // nibbles of columns 2b (low) and 2b+1 (high); masking each byte yields
  // the two int8 fragments of 16 * w (exact, the accumulator is shifted back
  // at the end).  Pair g covers tile columns 64 g .. 64 g + 63 of the wave:
  // fragment 2g holds the even ones, 2g+1 the odd ones (MFMA column l of
  // either is tile column 64 g + 2 l + parity).
  auto read_b4pair = [&](int sc, int kk, int g, v4i& even, v4i& odd) {
    const int r = kk * 32 + (lane >> 5) * 16 + ((lane & 15) >> 1);
    const int colb = wn * (WTN / 2) + g * 32 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
    const int8_t* a0 = sB + sc * B_BYTES + r * B_ROW + (((colb >> 4) ^ swzb(r)) << 4) + (colb & 15);
    const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(v2i))(a0));
    const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(v2i))(a0 + 8 * B_ROW));
    const v4i w = {lo.x, lo.y, hi.x, hi.y};
    even = (w << 4) & (int)0xF0F0F0F0;
    odd = w & (int)0xF0F0F0F0;
  };
  // read item r of a substep into fragment set (af, bf): A first, then B
  constexpr int NREAD = FM + (PACKED ? FN / 2 : FN);
  auto read_item = [&](auto r_, int sc, int kk, v4i (&af)[FM], v4i (&bf)[FN]) {
    constexpr int r = decltype(r_)::value;
    if constexpr (r < FM) read_a(sc, kk, r, af[r]);
    else if constexpr (PACKED) read_b4pair(sc, kk, r - FM, bf[2 * (r - FM)], bf[2 * (r - FM) + 1]);
    else read_b(sc, kk, r - FM, bf[r - FM]);
  };
  auto load_frags = [&](int sc, int kk, v4i (&af)[FM], v4i (&bf)[FN]) {
    static_for<0, NREAD>([&](auto r_) { read_item(r_, sc, kk, af, bf); });
  };
  // Copy items of one stage refill: the A copies, then the B copies --
  // int4 weights through registers take one register-load item first instead.
  constexpr int N_COPY = REGB4 ? A_INSTR + 1 : A_INSTR + B_INSTR;
  auto copy_item = [&](auto d_, int sc, int kt) {
    constexpr int d = decltype(d_)::value;
    if constexpr (REGB4) {
      if constexpr (d == 0) {
        fetch_b4(kt);
      } else {
        constexpr int q = d - 1;
        constexpr int slot_base = (q * NWAVES) * 64;
        const int sb = slot_base + wave * 64;
        if ((A_SLOTS % (NWAVES * 64)) == 0 || sb < A_SLOTS)
          lds_dma16_sv(a_base + (int64_t)kt * BK, a_off[q],
                       __builtin_amdgcn_readfirstlane(lds_addr(sA + sc * A_BYTES + sb * 16)));
      }
    } else if constexpr (d < A_INSTR) {
      const int sb = (d * NWAVES + wave) * 64;
      if ((A_SLOTS % (NWAVES * 64)) == 0 || sb < A_SLOTS)
        lds_dma16_sv(a_base + (int64_t)kt * BK, a_off[d],
                     __builtin_amdgcn_readfirstlane(lds_addr(sA + sc * A_BYTES + sb * 16)));
    } else {
      constexpr int q = d - A_INSTR;
      const int sb = (q * NWAVES + wave) * 64;
      if ((B_SLOTS % (NWAVES * 64)) == 0 || sb < B_SLOTS)
        lds_dma16_sv(b_base + (int64_t)kt * BK * (TB ? 1 : (PACKED ? n / 2 : n)), b_off[q],
                     __builtin_amdgcn_readfirstlane(lds_addr(sB + sc * B_BYTES + sb * 16)));
    }
  };
  // The MFMAs of one k-substep with other work spread between them: copy item
  // x of ND goes after MFMA x*NM/ND, read item x of NR after MFMA
  // x*(NM-2)/NR (the last two MFMAs cover the latency of the last reads).
  // Scheduling barriers pin this order, so that neither copies (which stall
  // issue while the address unit is busy) nor LDS reads bunch up in front of
  // the matrix core.
  // NB_: row blocks of the wave that hold rows of the tile (the MFMAs of
  // the others, all padding rows, are skipped; copies and reads stay).
  auto mfma_step = [&](v4i (&af)[FM], v4i (&bf)[FN], v16i (&acc)[FM][FN], auto ND_, auto NR_, auto&& copy, auto&& read,
                       auto NB_) {
    constexpr int NM = FM * FN, ND = decltype(ND_)::value, NR = decltype(NR_)::value, NB = decltype(NB_)::value;
    constexpr int RSPAN = NM > 2 ? NM - 2 : NM;
    static_for<0, NM>([&](auto m_) {
      constexpr int m = decltype(m_)::value;
      if constexpr (m / FN < NB)
        acc[m / FN][m % FN] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[m / FN], bf[m % FN], acc[m / FN][m % FN], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, ND>([&](auto d_) {
        if constexpr (decltype(d_)::value * NM / ND == m) {
          copy(d_);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
      static_for<0, NR>([&](auto r_) {
        if constexpr (decltype(r_)::value * RSPAN / NR == m) {
          read(r_);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    });
  };
  auto no_copy = [&](auto) {};

  // Entering stage j of the current tile: its copies are complete, and every
  // wave has finished reading stage j-1 (its fragments are in registers).
  // Stage 0 of a tile waits for everything (the previous tile's stores are
  // counted by the same counter).
  // Stage 0 of a tile: the previous tile's epilogue stores were issued after
  // this tile's prologue copies, and may stay in flight.  After an ordered
  // full-tile epilogue (FM*FN*16 separate stores, counted at half in case the
  // compiler pairs some) the wait allows that many more; after any other
  // epilogue only the later stages (younger than stage 0 either way).
  constexpr int FAST_STORES = COMBINE != kCombineAtomic ? FM * FN * (PACKED ? 4 : 8) : 0;
  constexpr int W0_FULL = (STAGES - 2) * LOADS_FULL + FAST_STORES < 63 ? (STAGES - 2) * LOADS_FULL + FAST_STORES : 63;
  constexpr int W0_SHORT = (STAGES - 2) * LOADS_SHORT + FAST_STORES < 63 ? (STAGES - 2) * LOADS_SHORT + FAST_STORES : 63;
  bool stores_counted = false;  // the previous epilogue took the ordered full-tile path
  auto sync_stage = [&](int j) {
    if (j + STAGES - 2 < ktiles) {
      if (j == 0 && stores_counted) {
        if (a_full) wait_vmcnt<W0_FULL>();
        else wait_vmcnt<W0_SHORT>();
      } else {
        if (a_full) wait_vmcnt<(STAGES - 2) * LOADS_FULL>();
        else wait_vmcnt<(STAGES - 2) * LOADS_SHORT>();
      }
    } else {
      wait_vmcnt<0>();
    }
    lds_barrier();
  };
  // After sync_stage(j): stage j+STAGES-1 may overwrite stage j-1's buffer.
  auto refill = [&](int j) {
    if (j + STAGES - 1 < ktiles) issue_stage((j + STAGES - 1) % STAGES, j + STAGES - 1);
  };

  // ---- epilogue of one tile.  Lane holds column lane%32 and rows
  // (r/4)*8 + (lane/32)*4 + r%4 of each 32x32 block; four consecutive
  // registers are four consecutive rows.  Returns whether the ordered
  // full-tile path (FM*FN*16 separate stores) was taken.
  auto epilogue = [&](const TileCoord& c, int pb, v16i (&acc)[FM][FN]) -> bool {
    // The tile coordinates pass through an opaque point so that no epilogue
    // address is computed (and kept live, or spilled) across the mainloop.
    int64_t e_row0 = uniform64(c.row0), e_col0 = uniform64(c.col0);
    int e_valid = __builtin_amdgcn_readfirstlane(c.valid_rows);
    asm volatile("" : "+s"(e_row0), "+s"(e_col0), "+s"(e_valid));
    // Likewise the lane and wave indices: every lane-dependent epilogue
    // address is computed here, not hoisted out of the tile loop (where it
    // would be kept live, or spilled, across the mainloop).
    int lane = lane_id;
    int wm = wave_m, wn = wave_n;
    asm volatile("" : "+v"(lane), "+s"(wm), "+s"(wn));
    const bool dump = p.acc_out != nullptr;
    // Whether this tile's rows go to y (the ordered reduce folds them) or
    // are added into out by atomics; per tile in the hybrid combine.
    const bool ord_tile =
        COMBINE == kCombineOrdered ||
        (COMBINE == kCombineHybrid && (int)((e_col0 / BN) % kHybridPeriod) >= p.hyb_atomic);
    // Tile-local column of this lane in MFMA block j (packed int4: block 2g
    // holds the even columns of pair g, block 2g+1 the odd ones).
    auto col_of = [&](int j) {
      return PACKED ? wn * WTN + (j >> 1) * 64 + 2 * (lane & 31) + (j & 1) : wn * WTN + j * 32 + (lane & 31);
    };
    float scv[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int cl = col_of(j);
      scv[j] = 1.0f;
      if (p.scale) {
        if (p.scale_bf16) {
          const uint32_t w = s_scale[pb][cl >> 1];
          scv[j] = __uint_as_float((cl & 1) ? (w & 0xFFFF0000u) : (w << 16));
        } else {
          scv[j] = __uint_as_float(s_scale[pb][cl]);
        }
      }
    }
    // Rows lr0 .. lr0+3 of the tile: their pertokenScale and logit (1.0
    // where absent, filled at the start), and in atomic mode their
    // destinations.
    auto row_factors = [&](int lr0, float4& P4, float4& L4) {
      P4 = *(const float4*)(&s_pts[pb][lr0]);
      L4 = *(const float4*)(&s_logit[pb][lr0]);
    };
    auto dests = [&](int lr0, int (&Dv)[4]) {
      if (!ord_tile) {
        // destination of each row from the raw rowIndex words; -1 when
        // outside [0, outputBS)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int r = lr0 + u;
          int64_t d;
          if (!p.row_index) d = e_row0 + r;
          else if (p.row_index_i32) d = (int32_t)s_ridx[pb][r];
          else d = (int64_t)((uint64_t)s_ridx[pb][2 * r] | ((uint64_t)s_ridx[pb][2 * r + 1] << 32));
          Dv[u] = (d >= 0 && d < p.output_bs) ? (int)d : -1;
        }
      } else {
        Dv[0] = Dv[1] = Dv[2] = Dv[3] = -1;
      }
    };
    auto first_row = [&](int i, int q) { return wm * WTM + i * 32 + q * 8 + (lane >> 5) * 4; };
    // One element: int32 -> fp32 (round to nearest even), then the three
    // factors in the oracle's order.
    auto value = [&](int i, int j, int r, float pv, float lv) {
      int32_t a = acc_elem<(FM * FN * 16 > 128)>(acc[i][j][r]);
      if constexpr (INT4) a >>= 4;  // weights were staged as 16 * w
      float v = (float)a;
      v = v * scv[j];
      v = v * pv;
      v = v * lv;
      return v;
    };
    // y stores: nontemporal, or through the caches when the reduce will read
    // a small y back from the MALL (kernels with two workgroups per CU only)
    const bool y_nt = OCC == 1 || !p.y_cached;
    auto store_y = [&](auto* ptr, auto v) {
      if (y_nt) __builtin_nontemporal_store(v, ptr);
      else *ptr = v;
    };
    const bool fast_epi = e_valid == BM && e_col0 + BN <= n && n < (int64_t(1) << 28) && !dump;
    if (fast_epi) {
      // Full tile: no per-element guards.  Ordered stores use one wave-uniform
      // row base and one 32-bit lane offset for every store (packed int4: the
      // even and odd blocks of a pair go out together, 8 bytes per lane).
      const uint32_t lane_off = (uint32_t)((lane >> 5) * 4 * n + (PACKED ? 2 : 1) * (lane & 31));
      float* wave_y = p.y + (e_row0 + wm * WTM) * n + e_col0 + wn * WTN;
      float* wave_out = p.out + e_col0 + wn * WTN + (PACKED ? 2 : 1) * (lane & 31);
      // the row factors of the next group of four rows are read one group
      // ahead, so no LDS wait sits between the stores
      float4 P_next, L_next;
      row_factors(first_row(0, 0), P_next, L_next);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lr0 = first_row(i, q);
          const float4 P4 = P_next, L4 = L_next;
          if (i * 4 + q + 1 < FM * 4) row_factors(first_row((i * 4 + q + 1) / 4, (i * 4 + q + 1) % 4), P_next, L_next);
          const float Pv[4] = {P4.x, P4.y, P4.z, P4.w}, Lv[4] = {L4.x, L4.y, L4.z, L4.w};
          int Dv[4];
          dests(lr0, Dv);
          if (ord_tile) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              float* rowp = wave_y + (int64_t)(i * 32 + q * 8 + u) * n;
              if constexpr (PACKED) {
                typedef float v2f __attribute__((ext_vector_type(2)));
#pragma unroll
                for (int g = 0; g < FN / 2; ++g)
                  store_y((v2f*)((rowp + g * 64) + lane_off),
                          v2f{value(i, 2 * g, q * 4 + u, Pv[u], Lv[u]), value(i, 2 * g + 1, q * 4 + u, Pv[u], Lv[u])});
              } else {
#pragma unroll
                for (int j = 0; j < FN; ++j) store_y((rowp + j * 32) + lane_off, value(i, j, q * 4 + u, Pv[u], Lv[u]));
              }
            }
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              if (Dv[u] < 0) continue;
              float* base = wave_out + (int64_t)Dv[u] * n;
#pragma unroll
              for (int j = 0; j < FN; ++j)
                __hip_atomic_fetch_add(base + (PACKED ? (j >> 1) * 64 + (j & 1) : j * 32),
                                       value(i, j, q * 4 + u, Pv[u], Lv[u]), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
    } else {
      // Partial tile (group tail or n tail) or accumulator dump: guarded.
      int64_t colj[FN];
      bool col_ok[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        colj[j] = e_col0 + col_of(j);
        col_ok[j] = colj[j] < n;
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lr0 = first_row(i, q);
          float4 P4, L4;
          row_factors(lr0, P4, L4);
          const float Pv[4] = {P4.x, P4.y, P4.z, P4.w}, Lv[4] = {L4.x, L4.y, L4.z, L4.w};
          int Dv[4];
          dests(lr0, Dv);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int lr = lr0 + u;
            if (lr >= e_valid) continue;
            float* base;
            if (ord_tile) {
              base = p.y + (e_row0 + lr) * n;
            } else {
              if (Dv[u] < 0) continue;
              base = p.out + (int64_t)Dv[u] * n;
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
              if (!col_ok[j]) continue;
              if (dump) {
                int32_t a = acc_elem<(FM * FN * 16 > 128)>(acc[i][j][q * 4 + u]);
                if constexpr (INT4) a >>= 4;
                p.acc_out[(e_row0 + lr) * n + colj[j]] = a;
              }
              const float v = value(i, j, q * 4 + u, Pv[u], Lv[u]);
              if (ord_tile)
                store_y(base + colj[j], v);
              else
                __hip_atomic_fetch_add(base + colj[j], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        }
      }
    }
    if constexpr (COMBINE == kCombineHybrid) return fast_epi && ord_tile;
    return fast_epi;
  };

  // ===== Continuous copy pipeline (int8 weights, at least STAGES k-steps).
  // One stream of k-steps across this workgroup's tiles: the refill issued
  // at a k-step fetches the k-slice STAGES steps ahead, which near a tile's
  // end belongs to the next tile, so no tile starts with a prologue wait.
  // Tile order is static: workgroup w takes the tiles of raster queue w % 8
  // (blocks of kTileBlock consecutive tiles dealt to the 8 queues in turn,
  // workgroups being dealt to the 8 XCDs in the same way) in turn with the
  // other workgroups of that queue.  Every k-step has the same shape: the
  // MFMAs of each substep but the last with the reads of the one after it;
  // the wait for the next k-step's copies and a barrier; the MFMAs of the
  // last substep with the refill of the buffer just released and the next
  // k-step's substep-0 reads.
  static_assert(KK % 2 == 0, "substeps alternate between two fragment sets");
  if constexpr (CONT) {
    {
      const int G = gridDim.x;
      const bool blocked = G % kTileQueues == 0;
      const int vq = blockIdx.x % kTileQueues, lw = blockIdx.x / kTileQueues, per_q = G / kTileQueues;
      auto tile_at = [&](int j) -> int {
        if (blocked) return queue_tile(vq, j * per_q + lw, total_tiles);
        const int64_t tt = (int64_t)j * G + blockIdx.x;
        return tt < total_tiles ? (int)tt : -1;
      };
      int j = 0;
      const int t0 = tile_at(0);
      if (t0 < 0) return;
      TileCoord cur = coord(t0);
      int t_nxt = tile_at(1);
      TileCoord nxt = cur;  // without a next tile the last refills re-copy this one
      if (t_nxt >= 0) nxt = coord(t_nxt);
      int pb = 0;
      dma_rows(cur, pb);
      set_sources(cur);
      static_for<0, STAGES>([&](auto st_) { issue_stage(decltype(st_)::value, decltype(st_)::value); });
      if (a_full) wait_vmcnt<(STAGES - 1) * LOADS_FULL>();
      else wait_vmcnt<(STAGES - 1) * LOADS_SHORT>();
      lds_barrier();
      v4i af[2][FM], bf[2][FN];
      // The k-steps run at a raised wave priority and the epilogue at the
      // base one: where the two workgroups of a CU share a SIMD, the one in
      // its k-loop issues its MFMAs and copies ahead of the other's epilogue.
      // Not for a workgroup's last two tiles, whose epilogues end the launch
      // (there the fair order finishes first).
      auto raise_priority = [&](int jj) {
        if (tile_at(jj + 2) >= 0) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      };
      raise_priority(0);
      load_frags(0, 0, af[0], bf[0]);
      int stage = 0;
      bool prev_fast = false;
      v16i acc[FM][FN];
      auto kstep = [&](int kt, int fill_ks, auto NB_) {
        const int stage_next = stage + 1 == STAGES ? 0 : stage + 1;
        // substeps 0 .. KK-2, each with the fragment reads of the next one
        static_for<0, KK - 1>([&](auto kk_) {
          constexpr int kk = decltype(kk_)::value;
          auto rd = [&](auto r_) { read_item(r_, stage, kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]); };
          mfma_step(af[kk & 1], bf[kk & 1], acc, std::integral_constant<int, 0>{}, std::integral_constant<int, NREAD>{},
                    no_copy, rd, NB_);
        });
        // the next k-step's copies have landed and every wave holds this
        // stage's fragments; after the first k-step of a tile the previous
        // tile's epilogue stores may still be in flight
        if (kt == 0 && prev_fast) {
          if (a_full) wait_vmcnt<W0_FULL>();
          else wait_vmcnt<W0_SHORT>();
        } else {
          if (a_full) wait_vmcnt<(STAGES - 2) * LOADS_FULL>();
          else wait_vmcnt<(STAGES - 2) * LOADS_SHORT>();
        }
        lds_barrier();
        auto cp = [&](auto d_) { copy_item(d_, stage, fill_ks); };
        auto rd0 = [&](auto r_) { read_item(r_, stage_next, 0, af[0], bf[0]); };
        mfma_step(af[(KK - 1) & 1], bf[(KK - 1) & 1], acc, std::integral_constant<int, N_COPY>{},
                  std::integral_constant<int, NREAD>{}, cp, rd0, NB_);
        stage = stage_next;
      };
      // The tile's k-steps.  With two workgroups per CU, a wave whose 32-row
      // blocks lie partly or wholly past the tile's valid rows (a group's
      // last tile) skips their MFMAs, which leaves the matrix core to the
      // other workgroup's waves on its SIMD (int4 workload GEMM -2.5%,
      // decode -1.2%; with one workgroup per CU it measured +0.4%).
      auto ksteps = [&](auto NB_) {
#pragma unroll 1
        for (int kt = 0; kt < ktiles - STAGES; ++kt) kstep(kt, kt + STAGES, NB_);
        set_sources(nxt);  // the remaining refills fetch the next tile's first k-slices
#pragma unroll 1
        for (int kt = ktiles - STAGES; kt < ktiles; ++kt) kstep(kt, kt + STAGES - ktiles, NB_);
      };
      while (true) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jj = 0; jj < FN; ++jj) acc[i][jj] = v16i{0};
        if constexpr (FM == 2 && OCC > 1) {
          const int live_rows = __builtin_amdgcn_readfirstlane(cur.valid_rows) - wave_m * WTM;  // wave-uniform
          if (live_rows > 32) ksteps(std::integral_constant<int, 2>{});
          else if (live_rows > 0) ksteps(std::integral_constant<int, 1>{});
          else ksteps(std::integral_constant<int, 0>{});
        } else {
          ksteps(std::integral_constant<int, FM>{});
        }
        // the next tile's row and column inputs go to the other buffer before
        // this tile's stores fill the copy queue
        if (t_nxt >= 0) dma_rows(nxt, pb ^ 1);
        __builtin_amdgcn_s_setprio(0);
        prev_fast = epilogue(cur, pb, acc);
        if (t_nxt < 0) break;
        ++j;
        raise_priority(j);
        cur = nxt;
        t_nxt = tile_at(j + 1);
        if (t_nxt >= 0) nxt = coord(t_nxt);
        pb ^= 1;
      }
      wait_vmcnt<0>();  // no copy in flight when the workgroup ends
      return;
    }
  }

  if constexpr (!CONT) {
  // ===== Tile-by-tile loop (int4 weights, or fewer than STAGES k-steps):
  // tiles from per-XCD queues (tiles running together on one XCD are
  // consecutive in raster order and share panels in its L2; an empty queue
  // steals from the others), each tile starting with its own prologue.
  if (tid == 0) {
    s_tiles[0] = grab_tile_from(p.tile_ctr, xcd, total_tiles);
    s_tiles[1] = s_tiles[0] >= 0 ? grab_tile_from(p.tile_ctr, xcd, total_tiles) : -1;
  }
  __syncthreads();
  int t = s_tiles[0];
  int t1 = s_tiles[1];
  if (t < 0) return;

  TileCoord cur = coord(t);
  int pb = 0;
  set_sources(cur);
  prologue();
  fetch_rows(cur);
  wait_vmcnt<0>();
  store_rows(pb);

  while (true) {
    // the tile after this one (t1) is known; the one after that is grabbed
    // now and read at the last stage, where all copies have landed anyway
    const bool has_next = t1 >= 0;
    TileCoord nxt = cur;
    if (has_next) nxt = coord(t1);

    v16i acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = v16i{0};

    sync_stage(0);
    refill(0);
    int pending = -1;
    if (tid == 0 && has_next) pending = atomicAdd(p.tile_ctr + xcd * kTileQueueStride, 1);
    // the next tile's row factors go to the other buffer at the last stage
    if (has_next) fetch_rows(nxt);
    v4i af[2][FM], bf[2][FN];
    load_frags(0, 0, af[0], bf[0]);

    int stage = 0;
    for (int kt = 0; kt < ktiles; ++kt) {
      const int stage_next = stage + 1 == STAGES ? 0 : stage + 1;
      static_for<0, KK>([&](auto kk_) {
        constexpr int kk = decltype(kk_)::value;
        constexpr int cur_f = kk & 1, nxt_f = cur_f ^ 1;
        if constexpr (kk + 1 < KK) {
          // next substep of this stage, read under this substep's MFMAs
          auto rd = [&](auto r_) {
            constexpr int r = decltype(r_)::value;
            if constexpr (r < FM) read_a(stage, kk + 1, r, af[nxt_f][r]);
            else read_b(stage, kk + 1, r - FM, bf[nxt_f][r - FM]);
          };
          mfma_step(af[cur_f], bf[cur_f], acc, std::integral_constant<int, 0>{},
                    std::integral_constant<int, FM + FN>{}, no_copy, rd, std::integral_constant<int, FM>{});
        } else {
          if constexpr (INT4) {
            // int4 weights fetched on entering this stage, for the stage
            // STAGES-1 ahead, go to LDS before the next fetch reuses b4reg
            if (kt + STAGES - 1 < ktiles) store_b4(stage == 0 ? STAGES - 1 : stage - 1);
          }
          const bool more = kt + 1 < ktiles;
          if (more) {
            sync_stage(kt + 1);
          } else {
            // last stage: every copy of this tile has landed (wait_vmcnt<0>
            // below covers the row loads and the queue grab too)
            wait_vmcnt<0>();
            if (has_next) store_rows(pb ^ 1);
            if (tid == 0) {
              int t2 = -1;
              if (has_next) {
                t2 = queue_tile(xcd, pending, total_tiles);
                if (t2 < 0) t2 = grab_tile_from(p.tile_ctr, xcd, total_tiles);
              }
              s_tiles[pb] = t2;
            }
            lds_barrier();  // every wave has its fragments; the next tile's copies may start
            if (has_next) {
              set_sources(nxt);
              prologue();
            }
          }
          // Under this substep's MFMAs: the refill of the buffer just
          // released (stage kt + STAGES) and the first substep of the next
          // stage.  One instruction stream for every case (wave-uniform
          // conditions inside the items), so that the accumulators stay in
          // the same registers whatever path a k-step takes.
          const bool fill = kt + STAGES < ktiles;
          const int kt_fill = kt + STAGES;
          const int sc_fill = stage;  // (kt + STAGES) % STAGES
          auto cp = [&](auto d_) {
            if (fill) copy_item(d_, sc_fill, kt_fill);
          };
          auto rd = [&](auto r_) {
            constexpr int r = decltype(r_)::value;
            if (more) {
              if constexpr (r < FM) read_a(stage_next, 0, r, af[nxt_f][r]);
              else read_b(stage_next, 0, r - FM, bf[nxt_f][r - FM]);
            }
          };
          __builtin_amdgcn_sched_barrier(0);
          mfma_step(af[cur_f], bf[cur_f], acc, std::integral_constant<int, N_COPY>{},
                    std::integral_constant<int, FM + FN>{}, cp, rd, std::integral_constant<int, FM>{});
        }
      });
      stage = stage_next;
    }
    const int t2 = s_tiles[pb];
    stores_counted = epilogue(cur, pb, acc);
    if (!has_next) break;
    t = t1;
    t1 = t2;
    cur = nxt;
    pb ^= 1;
  }
  }
}

// ---------------------------------------------------------------------------
// MxA8W4 GEMM ("aclnnGroupedMatmulFinalizeRoutingWeightNzV2", Atlas 350 notes
// on the MxA8W4 quantisation): x1 FP8 E4M3 (m,k); x2 FP4 E2M1 given
// transposed, (e,n,k) two per byte along k (low nibble = even k); E8M0 block
// scales, one per 32 k: pertokenScale (m, k/64, 2) for x1, scale
// (e, n, k/64, 2) for x2.  For row i of expert g:
//   acc[i][j] = sum_b 2^(sA[i][b]-127) * 2^(sB[g][j][b]-127) * sum_{k in b} x1[i][k] * w[k][j]
// accumulated in fp32 by v_mfma_scale_f32_32x32x64_f8f6f4, then
// y = acc * logit[i] and the same combine as the int8 path.
//
// Lane layout of that instruction (measured on the device): A lane l holds
// row l%32 with bytes 0-15 = k 16h..16h+15 and bytes 16-31 = k 32+16h..
// 32+16h+15 of the 64-k step (h = l/32); B lane l holds column l%32 with
// nibbles 0-31 = k 32h..32h+31; the scale operand of lane l is the block-h
// scale of its row (A) or column (B); the accumulator layout is that of the
// integer instruction (column l%32, rows (r/4)*8 + h*4 + r%4).
// ---------------------------------------------------------------------------
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// FP8 (B8 = true): the same kernel for FP8 E4M3 weights, given (e,n,k) or,
// with BKN, (e,k,n), with per-channel scale and per-token pertokenScale as in
// the int8 mode (no block scales; the instruction's scale operands are 1.0):
// acc is the fp32 sum and y = ((acc * scale) * pertokenScale) * logit.
// Measured on the device: with both operands FP8, B lane l holds column l%32
// with the byte layout of A.
// BM_ = 128 (NT = 256, two workgroups per CU) or 256 (NT = 512, eight waves
// of 64 x 128, one workgroup per CU); WN_ waves across the tile's columns;
// BK_ = 64, or 128 (FP8 only: two 64-k MFMA slices per stage, two stages).
template <int COMBINE, bool B8, bool BKN, int BM_ = 128, int NT = kThreads, int WN_ = 2, int BK_ = 64>
__global__ __launch_bounds__(NT, NT == kThreads ? 2 : 1) void mx_gemm_kernel(KParams p) {
  // BKN (FP8 only): weights given (e,k,n); a B stage then holds BK weight rows
  // of BN bytes, laid out and read with the int8 kernel's transpose reads
  static_assert(!BKN || B8, "the (e,k,n) weight layout is an FP8 mode");
  constexpr int BM = BM_, BN = 256, BK = BK_, STAGES = B8 ? (BK_ == 128 ? 2 : 3) : 4;
  static_assert(BK == 64 || (B8 && BK == 128), "128 k per stage: FP8 only");
  constexpr int KSUB = BK / 64;  // 64-k MFMA slices per stage
  constexpr int NWAVES = NT / 64;
  constexpr int WAVES_N = WN_, WAVES_M = NWAVES / WAVES_N;
  constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N, FM = WTM / 32, FN = WTN / 32;
  static_assert(WAVES_M * WAVES_N == NWAVES && FM >= 1 && FN >= 1 && WTM % 32 == 0 && WTN % 32 == 0,
                "waves cover the tile");
  constexpr int A_BYTES = BM * BK;         // fp8: one byte per k
  constexpr int B_COLB = B8 ? BK : BK / 2;  // fp8: 64 bytes per column and k-step; fp4: 32
  constexpr int B_BYTES = BN * B_COLB;
  constexpr int A_INSTR = A_BYTES / 16 / NT, B_INSTR = B_BYTES / 16 / NT;
  static_assert(A_INSTR >= 1 && B_INSTR >= 1 && A_INSTR * 16 * NT == A_BYTES && B_INSTR * 16 * NT == B_BYTES,
                "whole copies per thread");
  // Block-scale copies (MX): one dword per column (threads 0..BN-1) and per
  // row.  With 256 threads the rows' copies come from waves 0-1 on top of
  // their column copies; with 512 threads waves 4-7 copy the rows, so every
  // wave issues one scale copy per pair of slices.
  constexpr bool SC_SPLIT = NT == BM + BN;
  static_assert(B8 || SC_SPLIT || (NT == BN && BM <= NT), "scale copies cover the rows and columns");
  // Copies per thread and k-slice: A and B.  MX: a scale dword holds the
  // block scales of two k-slices, so even slices add one B-scale dword copy
  // per thread (waves 0-1 also an A-scale dword) into a ring of SC_SLOTS slots
  // of its own, indexed by the running count of slices.  A wait for a slice
  // allows the fewest copies its STAGES-2 younger slices can have issued.
  constexpr int LOADS_AB = A_INSTR + B_INSTR;
  constexpr int SC_LO = B8 ? 0 : (SC_SPLIT ? 1 : 2), SC_HI = B8 ? 0 : 1;
  constexpr int LOADS_LO = (STAGES - 2) * LOADS_AB + (STAGES - 2) / 2 * SC_LO;
  constexpr int LOADS_HI = (STAGES - 2) * LOADS_AB + (STAGES - 2) / 2 * SC_HI;
  constexpr int SC_SLOTS = B8 ? 1 : 4;
  static_assert(B8 || STAGES <= 5, "a scale slot is refilled only after its two k-slices are read");
  // When k is a multiple of 512 (a whole number of 8-slice groups), the four
  // scale dwords of 8 slices are copied at once, 16 bytes per row and per
  // column, with the group's first slice, into 2 slots of [row][4 dwords]; a
  // slot is refilled 6 slices after the group that used it ends.  Waits then
  // allow no scale copy among the younger slices.
  constexpr int G8_SLOTS = 2;
  constexpr int SC_WORDS = B8 ? 1 : (G8_SLOTS * 4 > SC_SLOTS ? G8_SLOTS * 4 : SC_SLOTS);
  constexpr int LOADS_G8 = (STAGES - 2) * LOADS_AB;

  __shared__ __attribute__((aligned(16))) int8_t sA[STAGES * A_BYTES];
  __shared__ __attribute__((aligned(16))) int8_t sB[STAGES * B_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t sSA[SC_WORDS][BM];  // the scale dwords of each row
  __shared__ __attribute__((aligned(16))) uint32_t sSB[SC_WORDS][BN];  // and of each column
  // per-row logit and (FP8) pertokenScale of a tile for its epilogue, as raw
  // words copied by the DMA path, double-buffered across consecutive tiles
  __shared__ __attribute__((aligned(16))) float s_lg[2][BM];
  __shared__ __attribute__((aligned(16))) float s_pt[2][BM];
  // FP8: the tile's per-column scale words (fp32: one per column; bf16: one
  // per column pair), double-buffered like the row factors
  __shared__ __attribute__((aligned(16))) uint32_t s_cs[2][B8 ? BN : 1];
  extern __shared__ __attribute__((aligned(16))) int32_t s_dyn[];
  int32_t* s_ends = s_dyn;
  int32_t* s_tile_pre = s_dyn + p.e;
  int64_t* s_scan = (int64_t*)sA;
  static_assert(STAGES * A_BYTES >= NT * 8, "scan scratch fits in the A stages");

  // an absent logit or pertokenScale reads as 1.0, a per-tensor
  // pertokenScale as its one value (filled once; the table build's barriers
  // publish the fill)
  const bool lg_rows = p.logit != nullptr;
  const bool pt_rows = B8 && p.pertoken != nullptr && !p.pertoken_scalar;
  {
    const float pt_fill = (B8 && p.pertoken && p.pertoken_scalar) ? p.pertoken[0] : 1.0f;
    for (int q = threadIdx.x; q < 2 * BM; q += NT) {
      if (!lg_rows) (&s_lg[0][0])[q] = 1.0f;
      if (!pt_rows) (&s_pt[0][0])[q] = pt_fill;
    }
  }
  build_group_table<NT>(p, BM, s_ends, s_tile_pre, s_scan);
  const int total_tiles = s_tile_pre[p.e];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, h = lane >> 5;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int64_t k = p.k, n = p.n;
  // MX with k % 64 == 32: the last k-step holds 32 valid k (its other half,
  // and that block's scale, read as zero products with a unit scale)
  const bool half_tail = !B8 && (k % BK) != 0;
  const int ktiles = (int)((k + BK - 1) / BK);
  const bool grp8 = !B8 && k % 512 == 0 && ktiles >= STAGES;  // (always the continuous pipeline)
  static_assert(B8 || STAGES <= 9, "a group's slot is refilled only after the group two before it is read");
  // MX: scale dwords per row or column; when k % 128 != 0 the block scales
  // come from copies padded to a whole dword (unit scales appended)
  const int64_t kdw = (k + 127) / 128;
  // waves that copy column (B) and row (A) scale dwords; lo_wave: both
  const bool b_sc_wave = wave * 64 < BN;
  const int a_sc_blk = SC_SPLIT ? wave - BN / 64 : wave;  // rows a_sc_blk*64 .. +63
  const bool a_sc_wave = a_sc_blk >= 0 && a_sc_blk * 64 < BM;
  const bool lo_wave = a_sc_wave && b_sc_wave;
  const uint32_t* sa_words = (const uint32_t*)p.pertoken;
  const uint32_t* sb_words = (const uint32_t*)p.scale;

  // copy sources of the current tile: wave-uniform bases, per-lane offsets (bytes)
  const int8_t* a_base = p.x1;
  const int8_t* b_base = (const int8_t*)p.x2;
  const uint32_t* sa_base = sa_words;
  const uint32_t* sb_base = sb_words;
  uint32_t a_off[A_INSTR], b_off[B_INSTR], sa_off = 0, sb_off = 0;
  // half-filled last k-step: per copy, whether this lane's chunk lies in the
  // missing half (it then fetches the chunk 32 k lower -- in bounds; its
  // products are cancelled by zeroed A bytes)
  uint32_t a_tail_mask = 0, b_tail_mask = 0;
  auto set_sources = [&](const TileCoord& c) {
    // The lane and wave indices pass through an opaque point: the per-lane
    // offsets are computed here for each tile, not hoisted out of the tile
    // loop (where they would stay live, or spill, across the k-loop).
    int lane = tid & 63, wave = tid >> 6, tid = threadIdx.x;
    asm volatile("" : "+v"(lane), "+v"(wave), "+v"(tid));
    a_base = (const int8_t*)uniform64((int64_t)(p.x1 + c.row0 * k));
    a_tail_mask = 0;
#pragma unroll
    for (int q = 0; q < A_INSTR; ++q) {
      const int slot = (q * NWAVES + wave) * 64 + lane;
      const int r = slot / (BK / 16), cpos = slot % (BK / 16);
      const int64_t row = min(c.row0 + r, p.m - 1);  // rows past the group: loaded, never stored
      a_off[q] = (uint32_t)((row - c.row0) * k + ((cpos ^ swz_a<BK>(r)) * 16));
      if ((cpos ^ swz_a<BK>(r)) >= 2) a_tail_mask |= 1u << q;
    }
    if constexpr (BKN) {
      // LDS chunk cpos of stage row r holds global chunk cpos ^ swz_b(r) of
      // that weight row (the int8 kernel's B layout); past n: loaded, never stored
      b_base = (const int8_t*)uniform64((int64_t)((const int8_t*)p.x2 + (int64_t)c.g * k * n + c.col0));
#pragma unroll
      for (int q = 0; q < B_INSTR; ++q) {
        const int slot = (q * NWAVES + wave) * 64 + lane;
        const int r = slot / (BN / 16), cpos = slot % (BN / 16);
        const int64_t colb = min(c.col0 + ((cpos ^ swz_b(r)) * 16), n - 16);
        b_off[q] = (uint32_t)((int64_t)r * n + (colb - c.col0));
      }
    } else {
      const int64_t colb = B8 ? k : k / 2;  // bytes of one weight column
      b_base = (const int8_t*)uniform64((int64_t)((const int8_t*)p.x2 + ((int64_t)c.g * n + c.col0) * colb));
      b_tail_mask = 0;
#pragma unroll
      for (int q = 0; q < B_INSTR; ++q) {
        const int slot = (q * NWAVES + wave) * 64 + lane;
        const int64_t cpr = B_COLB / 16;  // 16-byte chunks of a column per k-step
        const int r = slot / cpr, cpos = slot % cpr;
        const int64_t col = min(c.col0 + r, n - 1);    // columns past n: loaded, never stored
        // fp8 columns are stored and read like A rows (same swizzle); fp4
        // columns (two chunks) swap their chunks in every other group of 8
        // columns, so that 16 lanes reading 16 consecutive columns cover
        // all 64 banks (unswizzled, columns c and c + 8 share banks)
        const int gch = B8 ? (cpos ^ swz_a<BK>(r)) : (cpos ^ swz_b4(r));
        b_off[q] = (uint32_t)((col - c.col0) * colb + gch * 16);
        if (!B8 && gch == 1) b_tail_mask |= 1u << q;  // fp4: nibbles of k 32..63 of the step
      }
    }
    sa_base = (const uint32_t*)uniform64((int64_t)(sa_words + c.row0 * kdw));
    sa_off = (uint32_t)((min(c.row0 + (SC_SPLIT ? tid - BN : tid), p.m - 1) - c.row0) * kdw * 4);
    sb_base = (const uint32_t*)uniform64((int64_t)(sb_words + ((int64_t)c.g * n + c.col0) * kdw));
    sb_off = (uint32_t)((min(c.col0 + tid, n - 1) - c.col0) * kdw * 4);
  };
  // copies of k-slice kt (tile-local) into stage st; gs: the slice's running
  // count (8-slice groups: slot gs/8); pr: the running count of the scale
  // dwords issued before this slice's pair (its dword goes to ring slot pr --
  // counted per pair, not as gs/2, since a tile may hold an odd number of
  // slices)
  auto issue_stage = [&](int st, int kt, int gs, int pr) {
    // the half-filled last step: chunks of its missing half re-fetch the
    // valid half (every lane still issues its copy, so the waits' counts hold)
    const bool tail = half_tail && kt == ktiles - 1;  // wave-uniform
#pragma unroll
    for (int q = 0; q < A_INSTR; ++q)
      lds_dma16_sv(a_base + (int64_t)kt * BK, a_off[q] - ((tail && ((a_tail_mask >> q) & 1u)) ? 32u : 0u),
                   __builtin_amdgcn_readfirstlane(lds_addr(sA + st * A_BYTES + (q * NWAVES + wave) * 64 * 16)));
#pragma unroll
    for (int q = 0; q < B_INSTR; ++q)
      lds_dma16_sv(b_base + (int64_t)kt * (BKN ? (int64_t)BK * n : (int64_t)B_COLB),
                   b_off[q] - ((tail && ((b_tail_mask >> q) & 1u)) ? 16u : 0u),
                   __builtin_amdgcn_readfirstlane(lds_addr(sB + st * B_BYTES + (q * NWAVES + wave) * 64 * 16)));
    if constexpr (!B8) {
      if (grp8) {
        if ((kt & 7) == 0) {  // the four dwords of slices kt .. kt + 7, [row][4 dwords]
          const int slot = (gs >> 3) % G8_SLOTS;
          if (b_sc_wave)
            lds_dma16_sv(sb_base + kt / 2, sb_off,
                         __builtin_amdgcn_readfirstlane(lds_addr(&sSB[0][0] + (slot * BN + wave * 64) * 4)));
          if (a_sc_wave)
            lds_dma16_sv(sa_base + kt / 2, sa_off,
                         __builtin_amdgcn_readfirstlane(lds_addr(&sSA[0][0] + (slot * BM + a_sc_blk * 64) * 4)));
        }
      } else if ((kt & 1) == 0) {  // the dword holding the block scales of slices kt and kt + 1
        const int slot = pr % SC_SLOTS;
        if (b_sc_wave)
          lds_dma4_sv(sb_base + kt / 2, sb_off, __builtin_amdgcn_readfirstlane(lds_addr(&sSB[slot][wave * 64])));
        if (a_sc_wave)
          lds_dma4_sv(sa_base + kt / 2, sa_off,
                      __builtin_amdgcn_readfirstlane(lds_addr(&sSA[slot][a_sc_blk * 64])));
      }
    }
  };

  auto coord = [&](int tt) {
    TileCoord c = tile_coord<BM, BN>(p, s_ends, s_tile_pre, __builtin_amdgcn_readfirstlane(tt));
    c.g = __builtin_amdgcn_readfirstlane(c.g);
    c.valid_rows = __builtin_amdgcn_readfirstlane(c.valid_rows);
    c.row0 = uniform64(c.row0);
    c.col0 = uniform64(c.col0);
    return c;
  };

  // row factors of tile c into buffer pb: one word per row from the waves
  // covering rows 0..BM-1 (opaque indices, as in set_sources)
  auto dma_rows = [&](const TileCoord& c, int pb) {
    int tid = threadIdx.x, wave = tid >> 6;
    asm volatile("" : "+v"(tid), "+v"(wave));
    if constexpr (B8) {
      if (p.scale) {  // column scales: every wave, one word per lane (the last ones clamped)
        const int w = __builtin_amdgcn_readfirstlane(wave);
        const int words = p.scale_bf16 ? BN / 2 : BN;
        if (w * 64 < words) {
          const int64_t last = p.scale_bf16 ? (n - c.col0) / 2 - 1 : n - c.col0 - 1;  // last word inside n
          const uint32_t off = (uint32_t)(min((int64_t)tid, last) * 4);
          const void* base = p.scale_bf16 ? (const void*)((const uint16_t*)p.scale + (int64_t)c.g * n + c.col0)
                                          : (const void*)((const float*)p.scale + (int64_t)c.g * n + c.col0);
          lds_dma4_sv((const void*)uniform64((int64_t)base), off,
                      __builtin_amdgcn_readfirstlane(lds_addr(&s_cs[pb][w * 64])));
        }
      }
    }
    if (wave * 64 < BM) {
      const uint32_t off = (uint32_t)((min(c.row0 + tid, p.m - 1) - c.row0) * 4);
      const int w = __builtin_amdgcn_readfirstlane(wave);
      if (lg_rows)
        lds_dma4_sv((const void*)uniform64((int64_t)(p.logit + c.row0)), off,
                    __builtin_amdgcn_readfirstlane(lds_addr(&s_lg[pb][w * 64])));
      if (pt_rows)
        lds_dma4_sv((const void*)uniform64((int64_t)(p.pertoken + c.row0)), off,
                    __builtin_amdgcn_readfirstlane(lds_addr(&s_pt[pb][w * 64])));
    }
  };

  // one k-step on stage st (tile-local k-step kt): fragment reads, 8 MFMAs
  auto compute = [&](int st, int sub, int kt, int gs, int pr, v16f (&acc)[FM][FN]) {
    // E8M0 scale of this lane's block of row or column q: byte 2 (kt & 1) + h
    // of the scale dword in the ring slot of this slice's pair, or (8-slice
    // groups) of word (kt/2)%4 of the group's slot.  Read as one byte at a
    // lane part q * (bytes per row or column) + h plus a wave-uniform part.
    const int sc_qmul = grp8 ? 16 : 4;
    const int sc_kb = 2 * (kt & 1);
    const int sc_ua = grp8 ? ((gs >> 3) % G8_SLOTS) * BM * 16 + ((kt >> 1) & 3) * 4 + sc_kb
                           : (pr % SC_SLOTS) * BM * 4 + sc_kb;
    const int sc_ub = grp8 ? ((gs >> 3) % G8_SLOTS) * BN * 16 + ((kt >> 1) & 3) * 4 + sc_kb
                           : (pr % SC_SLOTS) * BN * 4 + sc_kb;
    const LDS_PTR(const uint8_t) sca = (const LDS_PTR(const uint8_t))(const void*)&sSA[0][0];
    const LDS_PTR(const uint8_t) scb = (const LDS_PTR(const uint8_t))(const void*)&sSB[0][0];
    auto sc_byte = [&](const LDS_PTR(const uint8_t) base, int u, int q) -> int { return base[q * sc_qmul + h + u]; };
    const int8_t* a_st = sA + st * A_BYTES;
    const int8_t* b_st = sB + st * B_BYTES;
    v8i af[FM];
    int sa[FM], sb[FN];
    const bool tail = half_tail && kt == ktiles - 1;  // k 32..63 of this step lie past k: zero A there
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WTM + i * 32 + (lane & 31);
      // slice sub of the stage: 16-byte chunks 4 sub + h and 4 sub + 2 + h of row r
      const v4i lo = *(const LDS_PTR(v4i))(a_st + r * BK + ((((sub << 2) | h) ^ swz_a<BK>(r)) << 4));
      v4i hi = *(const LDS_PTR(v4i))(a_st + r * BK + ((((sub << 2) | (2 + h)) ^ swz_a<BK>(r)) << 4));
      if (tail) hi = v4i{0, 0, 0, 0};
      af[i] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      sa[i] = B8 ? 127 : sc_byte(sca, sc_ua, r);
    }
    v8i bf[FN];
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) {
      const int cl = wn * WTN + jj * 32 + (lane & 31);
      if constexpr (BKN) {
        // two transpose reads per 16 k (as the int8 kernel's B fragment of one
        // k-substep); k 16h.. and 32+16h.. of column cl make the 32 bytes
        v4i half[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int r = sub * 64 + kk * 32 + h * 16 + ((lane & 15) >> 1);
          const int col = wn * WTN + jj * 32 + 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
          const int8_t* a0 = b_st + r * BN + (((col >> 4) ^ swz_b(r)) << 4) + (col & 15);
          const v2i lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(v2i))(a0));
          const v2i hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_PTR(v2i))(a0 + 8 * BN));  // same swizzle
          half[kk] = v4i{lo.x, lo.y, hi.x, hi.y};
        }
        bf[jj] = v8i{half[0].x, half[0].y, half[0].z, half[0].w, half[1].x, half[1].y, half[1].z, half[1].w};
        sb[jj] = 127;
      } else if constexpr (B8) {
        const v4i lo = *(const LDS_PTR(v4i))(b_st + cl * BK + ((((sub << 2) | h) ^ swz_a<BK>(cl)) << 4));
        const v4i hi = *(const LDS_PTR(v4i))(b_st + cl * BK + ((((sub << 2) | (2 + h)) ^ swz_a<BK>(cl)) << 4));
        bf[jj] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        sb[jj] = 127;
      } else {
        const v4i w = *(const LDS_PTR(v4i))(b_st + cl * B_COLB + ((h ^ swz_b4(cl)) << 4));
        bf[jj] = v8i{w.x, w.y, w.z, w.w, 0, 0, 0, 0};
        sb[jj] = sc_byte(scb, sc_ub, cl);
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int jj = 0; jj < FN; ++jj)
        acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[jj], acc[i][jj], 0, B8 ? 0 : 4, 0,
                                                                      sa[i], 0, sb[jj]);
  };

  // epilogue: y = acc * logit (FP8: ((acc * scale) * pertokenScale) * logit),
  // guarded by the tile's valid rows and n; row factors and column scales
  // from LDS buffer pb (no global load here: a compiler-inserted wait for one
  // would also wait for the next tile's copies in flight).  Returns whether
  // every lane issued all FM*FN*16 stores (an ordered full tile).
  auto epilogue = [&](const TileCoord& cc, int pb, v16f (&acc)[FM][FN]) -> bool {
    // tile coordinates and lane-dependent addresses are computed here
    // (opaque indices, as in set_sources)
    int64_t row0 = uniform64(cc.row0), col0 = uniform64(cc.col0);
    int valid = __builtin_amdgcn_readfirstlane(cc.valid_rows);
    int lane = threadIdx.x & 63, h = lane >> 5, wm = wave / WAVES_N, wn = wave % WAVES_N;
    asm volatile("" : "+s"(row0), "+s"(col0), "+s"(valid), "+v"(lane), "+v"(h), "+s"(wm), "+s"(wn));
    float col_scale[FN];
#pragma unroll
    for (int jj = 0; jj < FN; ++jj) {
      const int cl = wn * WTN + jj * 32 + (lane & 31);
      col_scale[jj] = 1.0f;
      if (B8 && p.scale) {
        if (p.scale_bf16) {
          const uint32_t w = s_cs[pb][cl >> 1];
          col_scale[jj] = __uint_as_float((cl & 1) ? (w & 0xFFFF0000u) : (w << 16));
        } else {
          col_scale[jj] = __uint_as_float(s_cs[pb][cl]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * WTM + i * 32 + (r / 4) * 8 + h * 4 + (r % 4);
        if (lr >= valid) continue;
        const int64_t row = row0 + lr;
        const float lg = s_lg[pb][lr];
        const float pt = s_pt[pb][lr];
        int64_t d = row;
        if constexpr (COMBINE == kCombineAtomic) {
          d = dest_row(p, row);
          if (d < 0) continue;
        }
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) {
          const int64_t col = col0 + wn * WTN + jj * 32 + (lane & 31);
          if (col >= n) continue;
          float v = acc[i][jj][r];
          if constexpr (B8) {  // ((acc * scale) * pertokenScale) * logit, each rounded
            v = v * col_scale[jj];
            v = v * pt;
          }
          v = v * lg;
          if constexpr (COMBINE == kCombineOrdered)
            __builtin_nontemporal_store(v, p.y + row * n + col);
          else
            __hip_atomic_fetch_add(p.out + d * n + col, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    return COMBINE == kCombineOrdered && valid == BM && col0 + BN <= n;
  };

  const int G = gridDim.x;
  const bool blocked = G % kTileQueues == 0;
  const int vq = blockIdx.x % kTileQueues, lw = blockIdx.x / kTileQueues, per_q = G / kTileQueues;
  auto tile_at = [&](int jj) -> int {
    if (blocked) return queue_tile(vq, jj * per_q + lw, total_tiles);
    const int64_t tt = (int64_t)jj * G + blockIdx.x;
    return tt < total_tiles ? (int)tt : -1;
  };
  // The k-steps run at a raised wave priority and the epilogue at the base
  // one (where the two workgroups of a CU share a SIMD, the one in its k-loop
  // issues first), except in a workgroup's last two tiles.
  auto raise_priority = [&](int jj) {
    if (tile_at(jj + 2) >= 0) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  };

  if (ktiles >= STAGES) {
    // Continuous copy pipeline: one stream of k-steps across the workgroup's
    // tiles.  The refill issued at a k-step fetches the k-slice STAGES-1
    // ahead, which near a tile's end is the next tile's (with its row
    // factors), so a tile starts without a prologue wait.  Without a next
    // tile the last refills copy this tile's first slices again (unused).
    int j = 0;
    const int t0 = tile_at(0);
    if (t0 >= 0) {
      TileCoord cur = coord(t0);
      int t_nxt = tile_at(1);
      TileCoord nxt = t_nxt >= 0 ? coord(t_nxt) : cur;
      int pb = 0;
      dma_rows(cur, pb);
      set_sources(cur);
      // running counts of slices issued and consumed (gfill, gstep) and of
      // scale pairs issued and consumed (pfill, puse: a pair starts at each
      // even tile-local slice)
      int gfill = 0, gstep = 0, pfill = 0, puse = 0;
#pragma unroll
      for (int st = 0; st < STAGES - 1; ++st) {
        if ((st & 1) == 0) ++pfill;
        issue_stage(st, st, gfill++, pfill - 1);
      }
      int stage = 0;
      bool prev_full = false;
      // After an ordered full-tile epilogue, its FM*FN*16 stores (issued
      // after the next tile's first slices) may stay in flight while stage 0
      // is awaited; after any other epilogue the plain wait also drains them.
      constexpr int FULL_STORES = FM * FN * 16;
      constexpr int W0_LO = LOADS_LO + FULL_STORES < 63 ? LOADS_LO + FULL_STORES : 63;
      constexpr int W0_HI = LOADS_HI + FULL_STORES < 63 ? LOADS_HI + FULL_STORES : 63;
      constexpr int W0_G8 = LOADS_G8 + FULL_STORES < 63 ? LOADS_G8 + FULL_STORES : 63;
      while (true) {
        raise_priority(j);
        v16f acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int jj = 0; jj < FN; ++jj) acc[i][jj] = v16f{0};
#pragma unroll 1
        for (int kt = 0; kt < ktiles; ++kt) {
          // this k-step's slice has landed; the STAGES-2 younger ones may still be in flight
          if (kt == 0 && prev_full) {
            if (grp8) wait_vmcnt<W0_G8>();
            else if (lo_wave) wait_vmcnt<W0_LO>();
            else wait_vmcnt<W0_HI>();
          } else if (grp8) {
            wait_vmcnt<LOADS_G8>();
          } else {
            if (lo_wave) wait_vmcnt<LOADS_LO>();
            else wait_vmcnt<LOADS_HI>();
          }
          lds_barrier();
          const int fill = kt + STAGES - 1;
          if (fill == ktiles) {  // from here on the refills are the next tile's
            set_sources(nxt);
            if (t_nxt >= 0) dma_rows(nxt, pb ^ 1);
          }
          const int fkt = fill < ktiles ? fill : fill - ktiles;
          if ((fkt & 1) == 0) ++pfill;
          issue_stage(stage == 0 ? STAGES - 1 : stage - 1, fkt, gfill, pfill - 1);
          ++gfill;
          if ((kt & 1) == 0) ++puse;
#pragma unroll
          for (int sub = 0; sub < KSUB; ++sub) compute(stage, sub, kt, gstep, puse - 1, acc);
          ++gstep;
          stage = stage + 1 == STAGES ? 0 : stage + 1;
        }
        __builtin_amdgcn_s_setprio(0);
        prev_full = epilogue(cur, pb, acc);
        if (t_nxt < 0) break;
        ++j;
        cur = nxt;
        pb ^= 1;
        t_nxt = tile_at(j + 1);
        nxt = t_nxt >= 0 ? coord(t_nxt) : cur;
      }
    }
  } else {
    // Tile by tile (k shorter than the pipeline): each tile starts with its
    // own prologue.
    for (int j = 0;; ++j) {
      const int t = tile_at(j);
      if (t < 0) break;
      const TileCoord c = coord(t);
      __syncthreads();  // every wave is done with the previous tile's stages and row factors
      raise_priority(j);
      dma_rows(c, 0);
      set_sources(c);
#pragma unroll
      for (int st = 0; st < STAGES - 1; ++st)
        if (st < ktiles) issue_stage(st, st, st, st / 2);
      v16f acc[FM][FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int jj = 0; jj < FN; ++jj) acc[i][jj] = v16f{0};
#pragma unroll 1
      for (int kt = 0; kt < ktiles; ++kt) {
        // stage kt complete; the stages issued after it may still be in flight
        if (kt + STAGES - 2 < ktiles) {
          if (lo_wave) wait_vmcnt<LOADS_LO>();
          else wait_vmcnt<LOADS_HI>();
        } else {
          wait_vmcnt<0>();
        }
        lds_barrier();
        if (kt + STAGES - 1 < ktiles)
          issue_stage((kt + STAGES - 1) % STAGES, kt + STAGES - 1, kt + STAGES - 1, (kt + STAGES - 1) / 2);
#pragma unroll
        for (int sub = 0; sub < KSUB; ++sub) compute(kt % STAGES, sub, kt, kt, kt / 2, acc);
      }
      __builtin_amdgcn_s_setprio(0);
      epilogue(c, 0, acc);
    }
  }
  wait_vmcnt<0>();  // no copy in flight when the workgroup ends
}

// ---------------------------------------------------------------------------
// MX block scales with k % 128 != 0: each row of `valid` scale bytes (k/32
// blocks) is copied into a row of `dst_row` bytes (a whole number of dwords),
// the bytes past the valid blocks set to 127 (a unit scale).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void mx_pad_scales_kernel(const uint8_t* src, uint8_t* dst, int64_t rows,
                                                                 int64_t src_row, int64_t dst_row, int64_t valid) {
  const int64_t total = rows * dst_row;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / dst_row, c = i % dst_row;
    dst[i] = c < valid ? src[r * src_row + c] : (uint8_t)127;
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
  if (blockIdx.x == 0 && threadIdx.x < (int)(kCtrlBytes / 4)) p.tile_ctr[threadIdx.x] = 0;
  // every column (atomic combine) or the atomic column tiles (hybrid)
  const int64_t ns = p.n4_seed, total = p.output_bs * ns;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * kThreads) {
    const int64_t d = idx / ns, j4 = hyb_col4(p, idx % ns, true);
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

// Zero the bucket counts and the GEMM's tile-queue counters.
__global__ __launch_bounds__(kThreads) void zero_counts_kernel(int32_t* counts, int64_t count, int32_t* ctrl) {
  if (blockIdx.x == 0 && threadIdx.x < (int)(kCtrlBytes / 4)) ctrl[threadIdx.x] = 0;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < count; i += (int64_t)gridDim.x * kThreads) counts[i] = 0;
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
// (nbins + 1 entries) and cursor := offsets, in chunks of 16384 counts.  Each
// thread takes 16 consecutive counts (four 16-byte loads when whole), scans
// them in registers, a shuffle scan over the wave and one LDS pass over the 16
// wave totals give its starting offset, and its 16 results go out as four
// 16-byte stores to each output.  (Sections of the workspace are 256-byte
// aligned and chunks start at multiples of 16 counts.)
constexpr int kScanPer = 16, kScanChunk = 1024 * kScanPer;
__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* counts, int32_t* offsets, int32_t* cursor, int64_t nbins) {
  __shared__ int32_t s_wave[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int32_t carry = 0;
  for (int64_t base = 0; base < nbins; base += kScanChunk) {
    const int64_t b0 = base + (int64_t)tid * kScanPer;
    const bool whole = b0 + kScanPer <= nbins;
    int32_t v[kScanPer];
    if (whole) {
#pragma unroll
      for (int q = 0; q < kScanPer / 4; ++q) {
        const int4 x = ((const int4*)(counts + b0))[q];
        v[4 * q] = x.x;
        v[4 * q + 1] = x.y;
        v[4 * q + 2] = x.z;
        v[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kScanPer; ++i) v[i] = b0 + i < nbins ? counts[b0 + i] : 0;
    }
    int32_t local = 0;  // exclusive scan within the thread
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      const int32_t c = v[i];
      v[i] = local;
      local += c;
    }
    int32_t incl = local;  // inclusive scan of the thread totals over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    if (lane == 63) s_wave[wv] = incl;
    __syncthreads();
    int32_t before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int32_t t = s_wave[w];
      before += w < wv ? t : 0;
      total += t;
    }
    const int32_t start = carry + before + incl - local;
    if (whole) {
#pragma unroll
      for (int q = 0; q < kScanPer / 4; ++q) {
        const int4 x = make_int4(start + v[4 * q], start + v[4 * q + 1], start + v[4 * q + 2], start + v[4 * q + 3]);
        ((int4*)(offsets + b0))[q] = x;
        ((int4*)(cursor + b0))[q] = x;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kScanPer; ++i)
        if (b0 + i < nbins) {
          offsets[b0 + i] = start + v[i];
          cursor[b0 + i] = start + v[i];
        }
    }
    carry += total;
    __syncthreads();  // s_wave is rewritten by the next chunk
  }
  if (tid == 0) offsets[nbins] = carry;
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

// out[d] = seed[d] + y[rows[0]] + y[rows[1]] + ... (left to right), rows in
// LDS in ascending order.  Rows in batches of kBatch: the batch's loads are
// issued together (independent, streamed once), then folded in ascending
// order; four float4 columns a kThreads apart per pass (32 loads in flight).
template <bool CACHED>
__device__ void fold_sorted_rows(const KParams& p, int64_t d, const int32_t* s_sorted, int len, int64_t j_lo,
                                 int64_t j_hi, bool from_out) {
  const int tid = threadIdx.x;
  const int64_t n = p.n;
  constexpr int kBatch = 8;
  typedef float v4f __attribute__((ext_vector_type(4)));
  constexpr int kCols = 4;
  for (int64_t jj0 = j_lo + tid; jj0 < j_hi; jj0 += kCols * kThreads) {
    v4f v[kCols];
    bool ok[kCols];
    int64_t jc[kCols];  // float4 column (the ordered columns' jj0 + c * kThreads-th)
#pragma unroll
    for (int c = 0; c < kCols; ++c) {
      ok[c] = jj0 + c * kThreads < j_hi;
      jc[c] = ok[c] ? hyb_col4(p, jj0 + c * kThreads, false) : 0;
      float4 sd = make_float4(0.f, 0.f, 0.f, 0.f);
      if (ok[c]) sd = from_out ? *((const float4*)(p.out + d * n) + jc[c]) : seed4(p, d, jc[c]);
      v[c] = v4f{sd.x, sd.y, sd.z, sd.w};
    }
    for (int s0 = 0; s0 < len; s0 += kBatch) {
      v4f yb[kBatch][kCols];
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (s0 + u < len) {
          const v4f* r = (const v4f*)(p.y + (int64_t)s_sorted[s0 + u] * n);
#pragma unroll
          for (int c = 0; c < kCols; ++c)
            if (ok[c]) yb[u][c] = CACHED ? r[jc[c]] : __builtin_nontemporal_load(r + jc[c]);
        }
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (s0 + u < len) {
#pragma unroll
          for (int c = 0; c < kCols; ++c)
            if (ok[c]) v[c] = v[c] + yb[u][c];
        }
    }
#pragma unroll
    for (int c = 0; c < kCols; ++c)
      if (ok[c]) __builtin_nontemporal_store(v[c], (v4f*)(p.out + d * n) + jc[c]);
  }
}

// The same fold for a destination with more than kSegMax rows: the covered
// rows are walked in ascending order, kSegMax at a time; each chunk's rows
// sent to d (found with a count per thread and a block-wide scan, so they
// come out ascending) are folded onto the running sum, which waits in out
// between chunks (the first chunk starts from the seed) -- the additions are
// the same, in the same order, as one fold over all the rows.  Each thread
// reads back only the out elements it wrote itself.
template <bool CACHED>
__device__ void fold_long_chunked(const KParams& p, int64_t d, int64_t covered, int32_t* s_rows, int32_t* s_wave,
                                  int64_t j_lo, int64_t j_hi) {
  constexpr int PER = kSegMax / kThreads;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  bool started = false;
  for (int64_t c0 = 0; c0 < covered; c0 += kSegMax) {
    const int64_t i0 = c0 + (int64_t)tid * PER;
    uint32_t hits = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (i0 + u < covered && dest_row(p, i0 + u) == d) hits |= 1u << u;
    const int mine = __popc(hits);
    int incl = mine;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    if (lane == 63) s_wave[wv] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      const int t = s_wave[w];
      before += w < wv ? t : 0;
      total += t;
    }
    int pos = before + incl - mine;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if ((hits >> u) & 1u) s_rows[pos++] = (int32_t)(i0 + u);
    __syncthreads();
    if (total > 0 || (!started && c0 + kSegMax >= covered)) {
      fold_sorted_rows<CACHED>(p, d, s_rows, total, j_lo, j_hi, started);
      started = true;
    }
    __syncthreads();  // s_rows and s_wave are rewritten by the next chunk
  }
}

// Work item w of an ordered reduce: destination w / reduce_split and its
// ordered float4 columns [lo, hi) (indices into the ordered columns, which
// are all columns unless hybrid), part w % reduce_split of the row.
struct FoldItem {
  int64_t d, lo, hi;
};
__device__ __forceinline__ FoldItem fold_item(const KParams& p, int64_t w) {
  const int64_t n4 = p.n4_ord, parts = p.reduce_split;
  const int64_t chunk = (n4 + parts - 1) / parts;
  FoldItem f;
  f.d = w / parts;
  f.lo = min(n4, (w % parts) * chunk);
  f.hi = min(n4, f.lo + chunk);
  return f;
}

// One work item (destination row, or a column range of it) per workgroup,
// grid-stride.  The destination's rows (unordered after the scatter) are
// ranked in LDS -- ranks are unique because row ids are -- then every column
// folds seed + y[rows] in ascending order.
__global__ __launch_bounds__(kThreads) void reduce_kernel(KParams p, const int32_t* offsets, const int32_t* list) {
  __shared__ int32_t s_src[kSegMax];
  __shared__ int32_t s_sorted[kSegMax];
  __shared__ int32_t s_wave[kThreads / 64];
  __shared__ int64_t s_red[kThreads];
  const int tid = threadIdx.x;
  int64_t covered = -1;
  for (int64_t w = blockIdx.x; w < p.output_bs * p.reduce_split; w += gridDim.x) {
    const FoldItem f = fold_item(p, w);
    const int64_t d = f.d;
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
      fold_sorted_rows<false>(p, d, s_sorted, len, f.lo, f.hi, false);
      __syncthreads();
    } else {
      if (covered < 0) covered = block_covered_rows(p, s_red);
      fold_long_chunked<false>(p, d, covered, s_sorted, s_wave, f.lo, f.hi);
    }
  }
}

// Ordered combine without a bucket index, for problems where every
// workgroup reading all of rowIndex is cheap (m * outputBS small): one
// workgroup per destination row (grid-stride) scans the covered rows in
// ascending order, kScanRows at a time (16 consecutive rows per thread, a
// count per thread, a block-wide exclusive scan of the counts), collects the
// rows sent to it -- already ascending -- and folds them like reduce_kernel.
constexpr int kScanPerThread = 16, kScanRows = kThreads * kScanPerThread;
template <bool CACHED>
__global__ __launch_bounds__(kThreads) void reduce_scan_kernel(KParams p) {
  __shared__ int32_t s_rows[kSegMax];
  __shared__ int32_t s_wave[kThreads / 64];
  __shared__ int64_t s_red[kThreads];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t covered = block_covered_rows(p, s_red);
  for (int64_t w = blockIdx.x; w < p.output_bs * p.reduce_split; w += gridDim.x) {
    const FoldItem f = fold_item(p, w);
    const int64_t d = f.d;
    int len = 0;  // rows found so far (the same in every thread)
    for (int64_t c0 = 0; c0 < covered; c0 += kScanRows) {
      const int64_t i0 = c0 + (int64_t)tid * kScanPerThread;
      uint32_t hits = 0;  // bit u: row i0 + u goes to d
      if (p.row_index && i0 + kScanPerThread <= covered) {
        // whole run of 16 rows: 16-byte loads, all issued before any compare
        // (i0 is a multiple of 16 and the base 16-byte aligned)
        if (p.row_index_i32) {
          uint4 w[kScanPerThread / 4];
#pragma unroll
          for (int q = 0; q < kScanPerThread / 4; ++q) w[q] = ((const uint4*)((const int32_t*)p.row_index + i0))[q];
#pragma unroll
          for (int q = 0; q < kScanPerThread / 4; ++q) {
            const uint32_t v[4] = {w[q].x, w[q].y, w[q].z, w[q].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) hits |= (uint32_t)((int64_t)(int32_t)v[t] == d) << (4 * q + t);
          }
        } else {
          uint4 w[kScanPerThread / 2];
#pragma unroll
          for (int q = 0; q < kScanPerThread / 2; ++q) w[q] = ((const uint4*)((const int64_t*)p.row_index + i0))[q];
#pragma unroll
          for (int q = 0; q < kScanPerThread / 2; ++q) {
            const int64_t lo = (int64_t)(((uint64_t)w[q].y << 32) | w[q].x);
            const int64_t hi = (int64_t)(((uint64_t)w[q].w << 32) | w[q].z);
            hits |= ((uint32_t)(lo == d) << (2 * q)) | ((uint32_t)(hi == d) << (2 * q + 1));
          }
        }
      } else {
#pragma unroll
        for (int u = 0; u < kScanPerThread; ++u)
          if (i0 + u < covered && dest_row(p, i0 + u) == d) hits |= 1u << u;
      }
      const int mine = __popc(hits);
      int incl = mine;  // inclusive scan over the wave
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      if (lane == 63) s_wave[wv] = incl;
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) {
        const int t = s_wave[w];
        before += w < wv ? t : 0;
        total += t;
      }
      int pos = len + before + incl - mine;
#pragma unroll
      for (int u = 0; u < kScanPerThread; ++u)
        if ((hits >> u) & 1u) {
          if (pos < kSegMax) s_rows[pos] = (int32_t)(i0 + u);
          ++pos;
        }
      len += total;
      __syncthreads();  // s_wave is rewritten by the next chunk
    }
    if (len <= kSegMax) {
      fold_sorted_rows<CACHED>(p, d, s_rows, len, f.lo, f.hi, false);
    } else {
      __syncthreads();  // every thread is done with this destination's first kSegMax rows
      fold_long_chunked<CACHED>(p, d, covered, s_rows, s_wave, f.lo, f.hi);
    }
    __syncthreads();  // s_rows is rewritten for the next destination
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
TileShape tile_shape(TileId id) {
  switch (id) {
    case kTile256x256: return {256, 256, 128};
    case kTile256x256k64:
    case kTileMx256: return {256, 256, 64};
    case kTileFp8x256k128: return {256, 256, 128};
    case kTile128x256i4: return {128, 256, 128};
    case kTile128x256: return {128, 256, 64};
    case kTile64x256: return {64, 256, 64};
    default: return {32, 256, 64};
  }
}

int tile_occupancy(TileId id) {
  return id == kTile256x256 || id == kTile256x256k64 || id == kTileMx256 || id == kTileFp8x256k128 ? 1 : 2;
}

int tile_stages(TileId id) {
  return id == kTile256x256 || id == kTile128x256i4 ? 2 : id == kTile256x256k64 ? 4 : 3;
}

// The 32-row tile serves groups of a few dozen rows, where the dynamic
// per-XCD queues of the tile-by-tile loop balance the uneven groups better.
bool uses_continuous_pipeline(bool int4, int64_t k, int bm, int bk, int stages) {
  (void)int4;
  return bm >= 64 && k / bk >= stages;
}

const char* tile_kernel_name(TileId id, bool int4, int64_t k, bool trans_b, bool mx, bool fp8) {
  const bool big = id == kTileMx256;
  if (mx) return big ? "mx_gemm_kernel<256,256,64,4x2,s4,fp8xfp4>" : "mx_gemm_kernel<128,256,64,2x2,s4,fp8xfp4>";
  if (fp8) {
    if (id == kTileFp8x256k128)
      return trans_b ? "mx_gemm_kernel<256,256,128,4x2,s2,fp8xfp8>" : "mx_gemm_kernel<256,256,128,4x2,s2,fp8xfp8,kn>";
    if (big) return trans_b ? "mx_gemm_kernel<256,256,64,4x2,s3,fp8xfp8>" : "mx_gemm_kernel<256,256,64,4x2,s3,fp8xfp8,kn>";
    return trans_b ? "mx_gemm_kernel<128,256,64,2x2,s3,fp8xfp8>" : "mx_gemm_kernel<128,256,64,2x2,s3,fp8xfp8,kn>";
  }
  // per tile: i8, i4, i8 cont, i4 cont, i8 transposed weights, i8 cont transposed weights
  static const char* names[kNumTiles][6] = {
      {"gmm_kernel<256,256,128,4x2,s2,i8>", "-", "gmm_kernel<256,256,128,4x2,s2,i8,cont>", "-",
       "gmm_kernel<256,256,128,4x2,s2,i8,tb>", "gmm_kernel<256,256,128,4x2,s2,i8,cont,tb>"},
      {"gmm_kernel<128,256,64,2x2,s3,i8>", "gmm_kernel<128,256,64,2x2,s3,i4>", "gmm_kernel<128,256,64,2x2,s3,i8,cont>",
       "gmm_kernel<128,256,64,2x2,s3,i4,cont>", "gmm_kernel<128,256,64,2x2,s3,i8,tb>",
       "gmm_kernel<128,256,64,2x2,s3,i8,cont,tb>"},
      {"gmm_kernel<64,256,64,1x4,s3,i8>", "gmm_kernel<64,256,64,1x4,s3,i4>", "gmm_kernel<64,256,64,1x4,s3,i8,cont>",
       "gmm_kernel<64,256,64,1x4,s3,i4,cont>", "gmm_kernel<64,256,64,1x4,s3,i8,tb>",
       "gmm_kernel<64,256,64,1x4,s3,i8,cont,tb>"},
      {"gmm_kernel<32,256,64,1x4,s3,i8>", "gmm_kernel<32,256,64,1x4,s3,i4>", "gmm_kernel<32,256,64,1x4,s3,i8,cont>",
       "gmm_kernel<32,256,64,1x4,s3,i4,cont>", "gmm_kernel<32,256,64,1x4,s3,i8,tb>",
       "gmm_kernel<32,256,64,1x4,s3,i8,cont,tb>"},
      {"gmm_kernel<256,256,64,4x2,s4,i8>", "gmm_kernel<256,256,64,4x2,s4,i4>", "gmm_kernel<256,256,64,4x2,s4,i8,cont>",
       "gmm_kernel<256,256,64,4x2,s4,i4,cont>", "gmm_kernel<256,256,64,4x2,s4,i8,tb>",
       "gmm_kernel<256,256,64,4x2,s4,i8,cont,tb>"},
      {"-", "-", "-", "-", "-", "-"},  // FP8 / MxA8W4 only
      {"-", "-", "-", "-", "-", "-"},  // FP8 only
      {"-", "gmm_kernel<128,256,128,2x2,s2,i4>", "-", "gmm_kernel<128,256,128,2x2,s2,i4,cont>", "-", "-"},
  };
  const TileShape ts = tile_shape(id);
  const bool cont = uses_continuous_pipeline(int4, k, ts.bm, ts.bk, tile_stages(id));
  if (trans_b && !int4) return names[(int)id][cont ? 5 : 4];
  return names[(int)id][(int4 ? 1 : 0) + (cont ? 2 : 0)];
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Workspace workspace_layout(int64_t m, int64_t n, int64_t output_bs, bool ordered, int64_t mx_pad_a,
                           int64_t mx_pad_b) {
  Workspace w{};
  size_t off = 0;
  w.ctrl_off = off;
  off += kCtrlBytes;
  w.mx_sa_off = off;
  off += align256((size_t)mx_pad_a);
  w.mx_sb_off = off;
  off += align256((size_t)mx_pad_b);
  if (ordered) {
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
  }
  w.total = off;
  return w;
}

// The continuous pipeline exists for tiles of at least 64 rows.  Variants
// built without int4 weights (I4 = false), or with int4 weights only
// (I8 = false), are never planned for the others.
template <int BM, int BN, int BK, int WM, int WN, int ST, int OCC, int COMB, int NT, bool I4, bool I8>
static void launch_gemm_mode(const KParams& kp, bool int4, bool trans_b, bool cont, dim3 gd, dim3 bd, size_t dyn,
                             hipStream_t s) {
  constexpr bool C = BM >= 64;
  if (int4) {
    if constexpr (I4) {
      if (C && cont) hipLaunchKernelGGL((gmm_kernel<BM, BN, BK, WM, WN, ST, OCC, true, COMB, C, false, NT>), gd, bd, dyn, s, kp);
      else hipLaunchKernelGGL((gmm_kernel<BM, BN, BK, WM, WN, ST, OCC, true, COMB, false, false, NT>), gd, bd, dyn, s, kp);
    }
  } else if constexpr (I8) {
    if (trans_b) {
      if (C && cont) hipLaunchKernelGGL((gmm_kernel<BM, BN, BK, WM, WN, ST, OCC, false, COMB, C, true, NT>), gd, bd, dyn, s, kp);
      else hipLaunchKernelGGL((gmm_kernel<BM, BN, BK, WM, WN, ST, OCC, false, COMB, false, true, NT>), gd, bd, dyn, s, kp);
    } else {
      if (C && cont) hipLaunchKernelGGL((gmm_kernel<BM, BN, BK, WM, WN, ST, OCC, false, COMB, C, false, NT>), gd, bd, dyn, s, kp);
      else hipLaunchKernelGGL((gmm_kernel<BM, BN, BK, WM, WN, ST, OCC, false, COMB, false, false, NT>), gd, bd, dyn, s, kp);
    }
  }
}

// The hybrid combine is compiled for the continuous pipeline of the tiles
// that plan it (HYB); the planner never picks it elsewhere.
template <int BM, int BN, int BK, int WM, int WN, int ST, int OCC, int NT = kThreads, bool I4 = true, bool I8 = true,
          bool HYB = false>
static void launch_gemm(const KParams& kp, bool int4, bool trans_b, int grid, hipStream_t s) {
  const dim3 gd(grid), bd(NT);
  const size_t dyn = ((size_t)(2 * kp.e + 1) * sizeof(int32_t) + 15) & ~(size_t)15;
  const bool cont = uses_continuous_pipeline(int4, kp.k, BM, BK, ST);
  if (kp.combine == kCombineOrdered) {
    launch_gemm_mode<BM, BN, BK, WM, WN, ST, OCC, kCombineOrdered, NT, I4, I8>(kp, int4, trans_b, cont, gd, bd, dyn, s);
  } else if (kp.combine == kCombineHybrid) {
    if constexpr (HYB && BM >= 64) {
      if (!cont) return;
      if (int4) {
        if constexpr (I4)
          hipLaunchKernelGGL((gmm_kernel<BM, BN, BK, WM, WN, ST, OCC, true, kCombineHybrid, true, false, NT>), gd, bd, dyn,
                             s, kp);
      } else if constexpr (I8) {
        if (trans_b)
          hipLaunchKernelGGL((gmm_kernel<BM, BN, BK, WM, WN, ST, OCC, false, kCombineHybrid, true, true, NT>), gd, bd, dyn,
                             s, kp);
        else
          hipLaunchKernelGGL((gmm_kernel<BM, BN, BK, WM, WN, ST, OCC, false, kCombineHybrid, true, false, NT>), gd, bd,
                             dyn, s, kp);
      }
    }
  } else {
    launch_gemm_mode<BM, BN, BK, WM, WN, ST, OCC, kCombineAtomic, NT, I4, I8>(kp, int4, trans_b, cont, gd, bd, dyn, s);
  }
}

bool hybrid_compiled(TileId id) { return id == kTile256x256 || id == kTile128x256 || id == kTile128x256i4; }

int64_t hybrid_cols4(int64_t n, int atomic_tiles, bool atomic_class) {
  const int64_t n4 = n / 4;
  int64_t cnt = 0;
  for (int64_t nt = 0; nt * 64 < n4; ++nt)
    if (((nt % kHybridPeriod) < atomic_tiles) == atomic_class) cnt += std::min<int64_t>(64, n4 - nt * 64);
  return cnt;
}

// Work items per destination row of the ordered reduce.  Destinations of
// more than kSegMax rows on average are folded in chunks, one serial chain
// of additions per column; their columns are then split over up to 16
// workgroups (kThreads float4 columns each), so that more chains run at once.
static int32_t ordered_reduce_split(int64_t m, int64_t output_bs, int64_t n) {
  if (output_bs <= 0 || m <= (int64_t)kSegMax * output_bs) return 1;
  return (int32_t)std::max<int64_t>(1, std::min<int64_t>(16, (n / 4) / kThreads));
}

int launch_all(const LaunchArgs& a, const Plan& plan, void* workspace, void* stream, void* const* gemm_events) {
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
  kp.pertoken_scalar = a.pertoken_scalar;
  kp.row_index_i32 = a.row_index_i32;
  kp.n_tiles_n = (int32_t)((a.n + ts.bn - 1) / ts.bn);
  kp.combine = plan.combine;
  const bool hybrid = plan.combine == kCombineHybrid;
  const bool ordered = plan.combine == kCombineOrdered || hybrid;  // y and the ordered reduce
  kp.hyb_atomic = hybrid ? plan.hybrid_atomic : 0;
  kp.n4_ord = hybrid ? hybrid_cols4(a.n, plan.hybrid_atomic, false) : a.n / 4;
  kp.n4_seed = hybrid ? hybrid_cols4(a.n, plan.hybrid_atomic, true) : a.n / 4;
  kp.reduce_split = ordered_reduce_split(a.m, a.output_bs, kp.n4_ord * 4);
  // a small y read back by the scan-lookup reduce (decode-sized problems)
  // goes through the caches and is found in the MALL: decode step -1.9%
  kp.y_cached = ordered && plan.scan_reduce && !a.mx && !a.fp8 && a.m * a.n * 4 <= kYCachedBytes;
  const MxPad mp = mx_pad(a.mx, a.m, a.k, a.n, a.e);
  const Workspace w = workspace_layout(a.m, a.n, a.output_bs, ordered, mp.a_bytes, mp.b_bytes);
  char* ws = (char*)workspace;
  kp.tile_ctr = (int32_t*)(ws + w.ctrl_off);
  if (mp.a_bytes > 0 && a.m > 0) {
    // block scales padded to whole dwords per row and column (unit scales appended)
    const int64_t src_row = 2 * ((a.k + 63) / 64), valid = a.k / 32;
    uint8_t* sa = (uint8_t*)(ws + w.mx_sa_off);
    uint8_t* sb = (uint8_t*)(ws + w.mx_sb_off);
    const int ga = (int)std::min<int64_t>(4096, (mp.a_bytes + kThreads - 1) / kThreads);
    const int gb = (int)std::min<int64_t>(4096, (mp.b_bytes + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(mx_pad_scales_kernel, dim3(ga), dim3(kThreads), 0, s, (const uint8_t*)a.pertoken, sa, a.m,
                       src_row, mp.row_bytes, valid);
    hipLaunchKernelGGL(mx_pad_scales_kernel, dim3(gb), dim3(kThreads), 0, s, (const uint8_t*)a.scale, sb,
                       (int64_t)a.e * a.n, src_row, mp.row_bytes, valid);
    kp.pertoken = (const float*)sa;
    kp.scale = sb;
  }

  // the tile-by-tile loop of the int8/int4 kernel takes its tiles from
  // queues whose counters start at zero; the other loops use a static order
  const bool dynamic_queues =
      !a.mx && !a.fp8 && !(ts.bm >= 64 && uses_continuous_pipeline(a.int4, a.k, ts.bm, ts.bk, tile_stages(plan.tile)));
  if (ordered && plan.scan_reduce) {
    kp.y = (float*)(ws + w.y_off);
    if (dynamic_queues)
      hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(kThreads), 0, s, (int32_t*)nullptr, (int64_t)0, kp.tile_ctr);
  } else if (ordered) {
    kp.y = (float*)(ws + w.y_off);
    int32_t* counts = (int32_t*)(ws + w.counts_off);
    int32_t* cursor = (int32_t*)(ws + w.cursor_off);
    int32_t* offsets = (int32_t*)(ws + w.offsets_off);
    int32_t* list = (int32_t*)(ws + w.list_off);
    const int gb = (int)std::min<int64_t>(1024, (a.output_bs + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(zero_counts_kernel, dim3(gb), dim3(kThreads), 0, s, counts, a.output_bs, kp.tile_ctr);
    if (a.m > 0) {
      const int gm = (int)std::min<int64_t>(2048, (a.m + kThreads - 1) / kThreads);
      hipLaunchKernelGGL(hist_kernel, dim3(gm), dim3(kThreads), 0, s, kp, counts);
      hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, counts, offsets, cursor, a.output_bs);
      hipLaunchKernelGGL(scatter_kernel, dim3(gm), dim3(kThreads), 0, s, kp, cursor, list);
    } else {
      hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, s, counts, offsets, cursor, a.output_bs);
    }
  }
  if (!ordered || hybrid) {  // out seeded where the GEMM adds by atomics
    const int gs = (int)std::min<int64_t>(4096, (a.output_bs * kp.n4_seed + kThreads - 1) / kThreads);
    hipLaunchKernelGGL(seed_kernel, dim3(gs > 0 ? gs : 1), dim3(kThreads), 0, s, kp);
  }
  if (a.m > 0 && plan.grid > 0) {
    if (gemm_events && gemm_events[0]) {
      const hipError_t er = hipEventRecord((hipEvent_t)gemm_events[0], s);
      if (er != hipSuccess) return (int)er;
    }
    const size_t dyn = ((size_t)(2 * kp.e + 1) * sizeof(int32_t) + 15) & ~(size_t)15;
    if (a.mx || a.fp8) {
      const int B = a.mx ? 0 : (a.trans_b ? 1 : 2);  // MxA8W4, FP8 (e,n,k), FP8 (e,k,n)
      const bool ord = kp.combine == kCombineOrdered;
      if (plan.tile == kTileFp8x256k128) {
        const dim3 gd(plan.grid), bd(512);
        if (B == 1) {
          if (ord) hipLaunchKernelGGL((mx_gemm_kernel<kCombineOrdered, true, false, 256, 512, 2, 128>), gd, bd, dyn, s, kp);
          else hipLaunchKernelGGL((mx_gemm_kernel<kCombineAtomic, true, false, 256, 512, 2, 128>), gd, bd, dyn, s, kp);
        } else if (B == 2) {
          if (ord) hipLaunchKernelGGL((mx_gemm_kernel<kCombineOrdered, true, true, 256, 512, 2, 128>), gd, bd, dyn, s, kp);
          else hipLaunchKernelGGL((mx_gemm_kernel<kCombineAtomic, true, true, 256, 512, 2, 128>), gd, bd, dyn, s, kp);
        }
      } else if (plan.tile == kTileMx256) {
        const dim3 gd(plan.grid), bd(512);
        if (B == 0) {
          if (ord) hipLaunchKernelGGL((mx_gemm_kernel<kCombineOrdered, false, false, 256, 512>), gd, bd, dyn, s, kp);
          else hipLaunchKernelGGL((mx_gemm_kernel<kCombineAtomic, false, false, 256, 512>), gd, bd, dyn, s, kp);
        } else if (B == 1) {
          if (ord) hipLaunchKernelGGL((mx_gemm_kernel<kCombineOrdered, true, false, 256, 512>), gd, bd, dyn, s, kp);
          else hipLaunchKernelGGL((mx_gemm_kernel<kCombineAtomic, true, false, 256, 512>), gd, bd, dyn, s, kp);
        } else {
          if (ord) hipLaunchKernelGGL((mx_gemm_kernel<kCombineOrdered, true, true, 256, 512>), gd, bd, dyn, s, kp);
          else hipLaunchKernelGGL((mx_gemm_kernel<kCombineAtomic, true, true, 256, 512>), gd, bd, dyn, s, kp);
        }
      } else {
        const dim3 gd(plan.grid), bd(kThreads);
        if (B == 0) {
          if (ord) hipLaunchKernelGGL((mx_gemm_kernel<kCombineOrdered, false, false>), gd, bd, dyn, s, kp);
          else hipLaunchKernelGGL((mx_gemm_kernel<kCombineAtomic, false, false>), gd, bd, dyn, s, kp);
        } else if (B == 1) {
          if (ord) hipLaunchKernelGGL((mx_gemm_kernel<kCombineOrdered, true, false>), gd, bd, dyn, s, kp);
          else hipLaunchKernelGGL((mx_gemm_kernel<kCombineAtomic, true, false>), gd, bd, dyn, s, kp);
        } else {
          if (ord) hipLaunchKernelGGL((mx_gemm_kernel<kCombineOrdered, true, true>), gd, bd, dyn, s, kp);
          else hipLaunchKernelGGL((mx_gemm_kernel<kCombineAtomic, true, true>), gd, bd, dyn, s, kp);
        }
      }
    } else switch (plan.tile) {
      case kTile256x256:
        launch_gemm<256, 256, 128, 4, 2, 2, 1, 512, false, true, true>(kp, a.int4, a.trans_b, plan.grid, s);
        break;
      case kTile256x256k64: launch_gemm<256, 256, 64, 4, 2, 4, 1, 512>(kp, a.int4, a.trans_b, plan.grid, s); break;
      case kTile128x256:
        launch_gemm<128, 256, 64, 2, 2, 3, 2, kThreads, true, true, true>(kp, a.int4, a.trans_b, plan.grid, s);
        break;
      case kTile128x256i4:
        launch_gemm<128, 256, 128, 2, 2, 2, 2, kThreads, true, false, true>(kp, a.int4, a.trans_b, plan.grid, s);
        break;
      case kTile64x256: launch_gemm<64, 256, 64, 1, 4, 3, 2>(kp, a.int4, a.trans_b, plan.grid, s); break;
      default: launch_gemm<32, 256, 64, 1, 4, 3, 2>(kp, a.int4, a.trans_b, plan.grid, s); break;
    }
    if (gemm_events && gemm_events[1]) {
      const hipError_t er = hipEventRecord((hipEvent_t)gemm_events[1], s);
      if (er != hipSuccess) return (int)er;
    }
  }
  if (ordered) {
    const int gr = (int)std::min<int64_t>(65535, a.output_bs * kp.reduce_split);
    if (plan.scan_reduce && kp.y_cached)
      hipLaunchKernelGGL(reduce_scan_kernel<true>, dim3(gr > 0 ? gr : 1), dim3(kThreads), 0, s, kp);
    else if (plan.scan_reduce)
      hipLaunchKernelGGL(reduce_scan_kernel<false>, dim3(gr > 0 ? gr : 1), dim3(kThreads), 0, s, kp);
    else
      hipLaunchKernelGGL(reduce_kernel, dim3(gr > 0 ? gr : 1), dim3(kThreads), 0, s, kp,
                         (const int32_t*)(ws + w.offsets_off), (const int32_t*)(ws + w.list_off));
  }
  return (int)hipGetLastError();
}

}  // namespace gmmfr
