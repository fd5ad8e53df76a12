// GEMM kernels of the NN layout for the four- and eight-wave 256x256 tiles, all four format pairs.
#include "gemm_kernel.h"

namespace fp8ds {

GemmFn gemm_fn_nn_large(int tile, int fa, int fb) { return pick_large<true, false>(tile, fa, fb); }

}  // namespace fp8ds
