// The fused GEMM pair kernels: a layer's dX (NN) and dW (TN) in one launch,
// for the 128x128 and 64x64 tiles (on 128-byte K units, and in the general kernel) and the
// eight-wave 256x256 tile, all four format pairs.
#include "gemm_kernel.h"

namespace fp8ds {

namespace {

template <int BM, int BN, int WGM, int WGN, int ST, int OCC>
GemmPairFn pick_pair(int fa, int fb) {
  if (fa == 0 && fb == 0) return gemm_pair_kernel<BM, BN, WGM, WGN, ST, OCC, true, false, false, false, 0, 0>;
  if (fa == 1 && fb == 0) return gemm_pair_kernel<BM, BN, WGM, WGN, ST, OCC, true, false, false, false, 1, 0>;
  if (fa == 0 && fb == 1) return gemm_pair_kernel<BM, BN, WGM, WGN, ST, OCC, true, false, false, false, 0, 1>;
  return gemm_pair_kernel<BM, BN, WGM, WGN, ST, OCC, true, false, false, false, 1, 1>;
}

GemmPairFn pick_pair_u128s(int fa, int fb) {
  if (fa == 0 && fb == 0) return gemm_pair_u128s_kernel<true, false, false, false, 0, 0>;
  if (fa == 1 && fb == 0) return gemm_pair_u128s_kernel<true, false, false, false, 1, 0>;
  if (fa == 0 && fb == 1) return gemm_pair_u128s_kernel<true, false, false, false, 0, 1>;
  return gemm_pair_u128s_kernel<true, false, false, false, 1, 1>;
}

GemmPairFn pick_pair_u128t(int fa, int fb) {
  if (fa == 0 && fb == 0) return gemm_pair_u128t_kernel<true, false, false, false, 0, 0>;
  if (fa == 1 && fb == 0) return gemm_pair_u128t_kernel<true, false, false, false, 1, 0>;
  if (fa == 0 && fb == 1) return gemm_pair_u128t_kernel<true, false, false, false, 0, 1>;
  return gemm_pair_u128t_kernel<true, false, false, false, 1, 1>;
}

}  // namespace

GemmPairFn gemm_pair_fn(int tile, int fa, int fb) {
  switch (tile) {
    case 7: return pick_pair_u128s(fa, fb);
    case 8: return pick_pair_u128t(fa, fb);
    case 1: return pick_pair<128, 128, 2, 2, 4, 2>(fa, fb);
    case 2: return pick_pair<64, 64, 2, 2, 4, 4>(fa, fb);
    default: return pick_pair<256, 256, 4, 2, 4, 1>(fa, fb);
  }
}

}  // namespace fp8ds
