// inst_skinny.hip -- instances of the skinny (M <= 32) streaming kernel for
// every (input type, output type) pair.
#include "tiles.hpp"
#include "skinny_gemm.hpp"

namespace tg {
namespace {

template <typename In, typename Out, int T>
constexpr KernelFn skinny_k() {
  constexpr SkinnyShape s = kSkinny[T];
  return &skinny_gemm_kernel<In, Out, s.mb, s.nblk, s.waves, s.unroll>;
}

}  // namespace

extern const KernelFn skinny_table[2][2][kNumSkinny];
// [input bf16/fp16][output fp32/same]
const KernelFn skinny_table[2][2][kNumSkinny] = {
    {{skinny_k<__bf16, float, 0>(), skinny_k<__bf16, float, 1>(), skinny_k<__bf16, float, 2>(),
      skinny_k<__bf16, float, 3>()},
     {skinny_k<__bf16, __bf16, 0>(), skinny_k<__bf16, __bf16, 1>(), skinny_k<__bf16, __bf16, 2>(),
      skinny_k<__bf16, __bf16, 3>()}},
    {{skinny_k<_Float16, float, 0>(), skinny_k<_Float16, float, 1>(), skinny_k<_Float16, float, 2>(),
      skinny_k<_Float16, float, 3>()},
     {skinny_k<_Float16, _Float16, 0>(), skinny_k<_Float16, _Float16, 1>(), skinny_k<_Float16, _Float16, 2>(),
      skinny_k<_Float16, _Float16, 3>()}}};
static_assert(kNumSkinny == 4, "update the skinny instance table");

}  // namespace tg
