// GEMM kernels of the NT layout for the 128x128, 64x64, 256x128 and 128x256 tiles, all four format pairs.
#include "gemm_kernel.h"

namespace fp8ds {

GemmFn gemm_fn_nt_small(int tile, int fa, int fb) { return pick_small<true, true>(tile, fa, fb); }

}  // namespace fp8ds
