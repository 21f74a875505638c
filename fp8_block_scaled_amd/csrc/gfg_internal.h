// Internal declarations shared by the host and device halves of libgfg.
#pragma once
#include <cstdint>

namespace gfg {
// Record a formatted message as the calling thread's last failure; returns code.
int fail(int code, const char* fmt, ...);
void clear_error();

// Tile-order settings of the GEMM launches (process-wide; set through
// grouped_fp8_set_tile_order): the number of XCDs the tile order is split
// over (8 by default) and the grouped-M width (0: each kernel's default).
int locality_num_xcd();
int locality_group_m();
// Output tile of the plain GEMM launches: 0 = chosen per launch, 1 = 128 x 256
// (128 x 128 where N is not a multiple of 256), 2 = 256 x 256.
int tile_shape_choice();
// Upper bound on the workgroups of a GEMM launch (0: one per CU).
int grid_limit();
}  // namespace gfg
