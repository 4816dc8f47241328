// internal.hpp -- layouts and kernel launchers shared by the library's own
// sources (api.hip, router.hip, lut.hip).  Nothing here is part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rvq {

// RVQ format ([FR] "Quantification et exactitude"): 3 stages, 256 entries, 8-wide vectors.
constexpr int kStages = 3;
constexpr int kCodes = 256;
constexpr int kVec = 8;

// Internal code layout of one RVQ matrix [rows][slices][3].
//
// The matrix is cut into tiles of kTileSlices input slices (one table lane
// per slice) and chunks of kChunkRows output rows.  A (tile, chunk) block is
// kChunkBytes contiguous bytes ordered [stage][half][lane][16]: byte i of lane
// (half h, lane l) of stage s is the stage-s code of row (chunk*32 + h*16 + i)
// and slice (tile*32 + l).  One wave64 load of 16 bytes per lane therefore
// reads 1 KB contiguous (one stage of one block).  Blocks are ordered
// tile-major: (tile * n_chunks + chunk).  Rows and slices beyond the matrix
// are zero codes whose table entries are zero (padded slices) or whose sums
// are never read (padded rows).
constexpr int kTileSlices = 32;
constexpr int kChunkRows = 32;
constexpr int kChunkBytes = kStages * kChunkRows * kTileSlices;  // 3072

struct MatGeom {
    int rows;       // output rows
    int slices;     // input slices (cols / 8)
    int n_tiles;    // ceil(slices / 32)
    int n_chunks;   // ceil(rows / 32)
    int64_t off;    // byte offset of the matrix inside an internal record
    int64_t bytes;  // n_tiles * n_chunks * 3072
};

struct Geometry {
    int d, ffn, E, k;
    MatGeom m[3];          // gate, up, down
    int64_t rec_int;       // internal record bytes
    int64_t rec_canon;     // canonical record bytes (9 d ffn / 8)
    int cb_dtype;          // 0 f32, 1 f16
    int64_t cb_bytes;      // one expert's codebooks: 3 * 3 * 256 * 8 * elem
    int ffn_pad;           // gate chunks * 32
    int d_pad;             // down chunks * 32
    int down_row_block;    // chunks per down workgroup
    int n_down_rb;         // down row blocks
};

Geometry make_geometry(int d, int ffn, int E, int k, int cb_dtype);

// Workspace of one handle (device memory, sized for max_tokens at open).
struct Workspace {
    double *tok_r;      // [T] RMS divisor (1.0 when no normalisation)
    double *route_part; // [T][n_rblk][E] fp64 partial logits
    float *part_gu;     // [T*k][2][n_tiles_in][ffn_pad] partial gate/up sums
    float *part_dn;     // [T*k][n_tiles_ffn][d_pad] partial down sums
    int *err;           // device error flag
    int n_rblk;         // router row blocks
};

constexpr int kRouterRows = 64;    // rows of W_r per router workgroup
constexpr int kRouterTok = 4;      // tokens per router workgroup
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;

// Launchers (all asynchronous on `s`; return hipError_t of the launch).
hipError_t launch_repack(const Geometry &g, const uint8_t *canon, uint8_t *internal, int n_experts,
                         hipStream_t s);
hipError_t launch_prep(const Geometry &g, const Workspace &w, const float *x, int T, int pre_rmsnorm,
                       double eps, hipStream_t s);
hipError_t launch_router(const Geometry &g, const Workspace &w, const float *x, const float *router_w,
                         int T, hipStream_t s);
hipError_t launch_topk(const Geometry &g, const Workspace &w, int T, int32_t *ids, float *gates,
                       hipStream_t s);
hipError_t launch_gateup(const Geometry &g, const Workspace &w, const uint8_t *codes, const void *cbs,
                         const float *x, const int32_t *ids, int T, hipStream_t s);
hipError_t launch_down(const Geometry &g, const Workspace &w, const uint8_t *codes, const void *cbs,
                       const int32_t *ids, int T, hipStream_t s);
hipError_t launch_combine(const Geometry &g, const Workspace &w, const float *x, const int32_t *ids,
                          const float *gates, float *y, int T, int residual, hipStream_t s);

}  // namespace rvq
