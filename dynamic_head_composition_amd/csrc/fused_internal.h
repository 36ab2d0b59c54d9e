// Internal interface between the fused-block C ABI (fused_api.cpp) and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ldc {

struct AttnArgs {
  int T, H;
  int window;             // the Lightweight DC window (its band: 8 blocks up to 113 keys, else 10)
  float scale;
  const void *q, *k, *v;
  const float* g;         // Lightweight DC scale G [T,H] (with the band)
  const uint32_t* band;   // composed-map band of the Lightweight DC score pass, or null
  const int32_t* rs;      // run start of every token
  const int32_t* order;   // the (128-query) tiles, most stages first
  float* o;
};

// 1024-token blocks of the run-start pass (one int of workspace each).
size_t run_blocks(int64_t T);
// Ints of the item-order area: a histogram and cursors of the tiles' stage
// counts, then one int per 128-query tile.
size_t order_ints(int64_t T);
// rs[t] = first token of the run of equal ids holding t (`last`: run_blocks(T)
// ints), and the tiles ordered by their stage count, most first (`order`:
// order_ints(T) ints; the tile list starts at order + order_list_offset()).
hipError_t run_starts_dispatch(const int32_t* doc, int T, int* last, int* rs, int* order, hipStream_t st);
int order_list_offset();
// ldc = false: the main attention alone (a.band, a.g unused).
hipError_t attn_fwd_dispatch(int d, const AttnArgs& a, bool ldc, hipStream_t st);

}  // namespace ldc
