// Internal interface between the host planner (gmmfr_api.cpp) and the HIP
// kernels (gmmfr_kernels.hip).  Not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace gmmfr {

constexpr int kMaxExperts = 1024;

// kCombineHybrid: of every kHybridPeriod consecutive 256-column tiles, the
// first Plan::hybrid_atomic are combined by atomics from the GEMM epilogue
// and the others through y and the ordered reduce (an unspecified order of
// additions, like the atomic mode).
enum Combine : int32_t { kCombineAtomic = 1, kCombineOrdered = 2, kCombineHybrid = 3 };
constexpr int kHybridPeriod = 8;

// GEMM tile variants compiled into the library.
enum TileId : int32_t {
  kTile256x256 = 0,     // BM=256 BN=256 BK=128, 4x2 waves of 64x128 (512 threads), 2 stages, 1 workgroup
                        // per CU; int8 weights and k % 128 == 0 only
  kTile128x256 = 1,     // BM=128 BN=256, 2x2 waves of 64x128, 3 stages
  kTile64x256 = 2,      // BM=64  BN=256, 1x4 waves of 64x64, 3 stages
  kTile32x256 = 3,      // BM=32  BN=256, 1x4 waves of 32x64, 3 stages
  kTile256x256k64 = 4,  // BM=256 BN=256 BK=64, 4x2 waves of 64x128 (512 threads), 4 stages, 1 workgroup per CU
  kTileMx256 = 5,       // FP8 / MxA8W4: BM=256 BN=256 BK=64, 4x2 waves of 64x128 (512 threads), 1 workgroup
                        // per CU (the FP8 kernels' other tile is kTile128x256)
  kTileFp8x256k128 = 6, // FP8 with k % 128 == 0: as kTileMx256 with BK=128, 2 stages
  kTile128x256i4 = 7,   // int4 weights with k % 128 == 0: as kTile128x256 with BK=128, 2 stages
  kNumTiles = 8
};

struct TileShape {
  int32_t bm, bn, bk;
};
TileShape tile_shape(TileId id);

// Everything a launch needs; pointers are device addresses.
struct LaunchArgs {
  const int8_t* x1;
  const void* x2;            // int8 (e,k,n), int8 (e,n,k) when trans_b, or packed int4 (e,k,n/8) words
  const void* scale;         // f32 / bf16 (e,1,n) or nullptr
  const float* pertoken;     // (m), (1) when pertoken_scalar, or nullptr
  const float* logit;        // (m) or nullptr
  const int64_t* group_list; // (e)
  const void* row_index;     // int64 / int32 (m) or nullptr (identity)
  const uint16_t* shared;    // bf16 (bsdp,n) or nullptr
  float* out;                // (output_bs,n)
  int32_t* acc_out;          // (m,n) or nullptr
  int64_t m, k, n;
  int32_t e;
  int32_t group_list_type;
  int32_t scale_bf16;
  int32_t pertoken_scalar;   // one pertokenScale value for every row
  int32_t row_index_i32;
  int32_t int4;
  int32_t trans_b;           // int8 weights given as (e,n,k)
  int32_t mx;                // MxA8W4: x1 fp8 e4m3, x2 fp4 e2m1 (e,n,k/2 bytes), scale/pertoken E8M0 block scales
  int32_t fp8;               // x1 fp8 e4m3, x2 fp8 e4m3 (e,n,k), scale fp32/bf16 (e,1,n), pertoken fp32 (m)
  int64_t bsdp, shared_offset, output_bs;
};

// Workspace carve-up (byte offsets, 256-aligned).  Every plan has the control
// block (GEMM tile-queue counters); the ordered combine adds the rest.
constexpr size_t kCtrlBytes = 1024;
struct Workspace {
  size_t ctrl_off, mx_sa_off, mx_sb_off, y_off, counts_off, cursor_off, offsets_off, list_off, total;
};
// MxA8W4 with k % 128 != 0: the block scales are copied into the workspace,
// each row padded to k rounded up to 128 (whole dwords of four block scales).
struct MxPad {
  int64_t row_bytes;        // bytes per padded row (0 when no padding)
  int64_t a_bytes, b_bytes; // padded copies of pertokenScale (m rows) and scale (e*n rows)
};
inline MxPad mx_pad(bool mx, int64_t m, int64_t k, int64_t n, int64_t e) {
  if (!mx || k % 128 == 0) return MxPad{0, 0, 0};
  const int64_t row = (k + 127) / 128 * 4;
  return MxPad{row, m * row, e * n * row};
}
Workspace workspace_layout(int64_t m, int64_t n, int64_t output_bs, bool ordered, int64_t mx_pad_a = 0,
                           int64_t mx_pad_b = 0);

struct Plan {
  Combine combine;
  TileId tile;
  int32_t grid;             // GEMM workgroups (persistent)
  bool scan_reduce;         // ordered combine without the bucket index (small m * outputBS)
  int32_t hybrid_atomic;    // kCombineHybrid: atomic column tiles in each kHybridPeriod (1 .. period-1)
  size_t workspace_bytes;
};

// The ordered combine scans rowIndex once per destination instead of
// building a bucket index when m * outputBS is at most this.
constexpr int64_t kScanReduceMax = int64_t(1) << 23;

// Enqueue the whole computation.  Returns 0 or a hipError_t value.
// gemm_events: optional {start, stop} hipEvent_t recorded around the GEMM.
int launch_all(const LaunchArgs& a, const Plan& plan, void* workspace, void* stream, void* const* gemm_events);

// Workgroups per CU the GEMM variant is compiled for, and its LDS stages.
int tile_occupancy(TileId id);
int tile_stages(TileId id);
// Whether the GEMM runs the continuous copy pipeline (int8 weights, tiles of
// at least 64 rows and at least `stages` k-steps per tile) rather than the
// tile-by-tile loop.
bool uses_continuous_pipeline(bool int4, int64_t k, int bm, int bk, int stages);
// Tiles whose continuous pipeline is compiled with the hybrid combine.
bool hybrid_compiled(TileId id);
// Float4 columns in the atomic (or the ordered) column tiles of a hybrid plan.
int64_t hybrid_cols4(int64_t n, int atomic_tiles, bool atomic_class);
const char* tile_kernel_name(TileId id, bool int4, int64_t k, bool trans_b, bool mx, bool fp8);

}  // namespace gmmfr
