// Internal interface between the host planner (gmmfr_api.cpp) and the HIP
// kernels (gmmfr_kernels.hip).  Not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace gmmfr {

constexpr int kMaxExperts = 1024;

enum Combine : int32_t { kCombineAtomic = 1, kCombineOrdered = 2 };

// GEMM tile variants compiled into the library.
enum TileId : int32_t {
  kTile256x256 = 0,   // BM=256 BN=256, 2x2 waves of 128x128, 3 stages, 1 workgroup per CU
  kTile128x256 = 1,   // BM=128 BN=256, 2x2 waves of 64x128, 3 stages
  kTile64x256 = 2,    // BM=64  BN=256, 1x4 waves of 64x64, 3 stages
  kTile32x256 = 3,    // BM=32  BN=256, 1x4 waves of 32x64, 3 stages
  kNumTiles = 4
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
  size_t ctrl_off, y_off, counts_off, cursor_off, offsets_off, list_off, total;
};
Workspace workspace_layout(int64_t m, int64_t n, int64_t output_bs, bool ordered);

struct Plan {
  Combine combine;
  TileId tile;
  int32_t grid;             // GEMM workgroups (persistent)
  size_t workspace_bytes;
};

// Enqueue the whole computation.  Returns 0 or a hipError_t value.
// gemm_events: optional {start, stop} hipEvent_t recorded around the GEMM.
int launch_all(const LaunchArgs& a, const Plan& plan, void* workspace, void* stream, void* const* gemm_events);

// Workgroups per CU the GEMM variant is compiled for.
int tile_occupancy(TileId id);
// Whether the GEMM runs the continuous copy pipeline (int8 weights, tiles of
// at least 64 rows and at least `stages` k-steps per tile) rather than the
// tile-by-tile loop.
bool uses_continuous_pipeline(bool int4, int64_t k, int bm, int bk, int stages);
const char* tile_kernel_name(TileId id, bool int4, int64_t k, bool trans_b, bool mx, bool fp8);

}  // namespace gmmfr
