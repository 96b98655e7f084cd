// nf4_gemm.h -- the matrix-core NF4 W4A16 product (private to libnf4).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "nf4.h"

namespace nf4gemm {

// Launch shape: MT row tiles of 16 and 64 NT columns per workgroup, gx x gy
// workgroups over columns and rows, SK splits of the K blocks; ws_bytes of
// workspace used.
struct Plan {
  int MT, NT, SK;
  int64_t gx, gy;
  size_t ws_bytes;
};

// The plan for an M x N x K product given ws_avail bytes of workspace.
Plan plan(int64_t M, int64_t N, int64_t K, size_t ws_avail);

// Launches the product (fast-path shapes only; see nf4_gemm).
nf4_status launch(const uint8_t* packed, const uint8_t* absmax_q, const uint16_t* absmax2,
                  const uint16_t* code2, float offset, int64_t M, int64_t N, int64_t K, int lbs,
                  int ls2, const uint16_t* x, uint16_t* y, void* ws, size_t ws_bytes,
                  hipStream_t st);

}  // namespace nf4gemm
