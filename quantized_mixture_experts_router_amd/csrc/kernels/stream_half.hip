// Launchers of the weight-streaming grouped GEMM (stream_kernel.hpp) for
// tiles of 8 rows: one-stage launches of 1, 4 or 8 items a stage (256, 1024
// or 2048 codes at 4 bits; 128, 512 or 1024 at 8), built apart from the
// 16-row launchers so that the two compile in parallel.
#include "stream_kernel.hpp"

namespace qmoe {

namespace {

template <int BITS, bool FC1, int HS>
hipError_t pick_rb(int rb, const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  if (rb == 2) return pick_scale<BITS, 1, FC1, true, 2, HS>(g, grid, lds, st);
  return pick_scale<BITS, 1, FC1, true, 1, HS>(g, grid, lds, st);
}

template <int BITS, bool FC1>
hipError_t pick_hs(int rb, int hs, const GemmArgs& g, dim3 grid, size_t lds, hipStream_t st) {
  switch (hs) {
    case 1: return pick_rb<BITS, FC1, 1>(rb, g, grid, lds, st);
    case 4: return pick_rb<BITS, FC1, 4>(rb, g, grid, lds, st);
    case 8: return pick_rb<BITS, FC1, 8>(rb, g, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_stream_half(int bits, bool fc1, int rb, int hs, const GemmArgs& g, dim3 grid, size_t lds,
                              hipStream_t st) {
  if (bits == 4) return fc1 ? pick_hs<4, true>(rb, hs, g, grid, lds, st) : pick_hs<4, false>(rb, hs, g, grid, lds, st);
  return fc1 ? pick_hs<8, true>(rb, hs, g, grid, lds, st) : pick_hs<8, false>(rb, hs, g, grid, lds, st);
}

}  // namespace qmoe
