// GEMM kernels of the NT layout for the four- and eight-wave 256x256 tiles, all four format pairs.
#include "gemm_kernel.h"

namespace fp8ds {

GemmFn gemm_fn_nt_large(int tile, int fa, int fb) { return pick_large<true, true>(tile, fa, fb); }

}  // namespace fp8ds
