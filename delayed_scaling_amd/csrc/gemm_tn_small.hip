// GEMM kernels of the TN layout for the 128x128, 64x64, 256x128 and 128x256 tiles, all four format pairs.
#include "gemm_kernel.h"

namespace fp8ds {

GemmFn gemm_fn_tn_small(int tile, int fa, int fb) { return pick_small<false, false>(tile, fa, fb); }

}  // namespace fp8ds
