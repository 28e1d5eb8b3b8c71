// Instantiations of the W4A16 GEMM kernel (gemm_w4_kernel.h) for 3 token tile(s) of 16.
#include "gemm_w4_kernel.h"

namespace ss {
void launch_w4_tt3(const W4Params& p, int tpw, int epi, bool tiled, int G, hipStream_t st) {
  w4::launch_tt<3>(p, tpw, epi, tiled, G, st);
}
}  // namespace ss
