// inst_skinny.hip -- instances of the skinny (M <= 32) streaming kernel for
// every (input type, output type) pair and every shape in kSkinny.
#include <array>
#include <utility>

#include "tiles.hpp"
#include "skinny_gemm.hpp"

namespace tg {
namespace {

template <typename In, typename Out, int T>
constexpr KernelFn skinny_k() {
  constexpr SkinnyShape s = kSkinny[T];
  return &skinny_gemm_kernel<In, Out, s.mb, s.nb, s.waves, s.stages, s.sk>;
}

template <typename In, typename Out, std::size_t... I>
constexpr std::array<KernelFn, sizeof...(I)> skinny_array(std::index_sequence<I...>) {
  return {skinny_k<In, Out, I>()...};
}
template <typename In, typename Out>
constexpr std::array<KernelFn, kNumSkinny> row() {
  return skinny_array<In, Out>(std::make_index_sequence<kNumSkinny>{});
}

}  // namespace

// [input bf16/fp16][output fp32/same][shape]
extern const std::array<KernelFn, kNumSkinny> skinny_table[2][2];
const std::array<KernelFn, kNumSkinny> skinny_table[2][2] = {{row<__bf16, float>(), row<__bf16, __bf16>()},
                                                            {row<_Float16, float>(), row<_Float16, _Float16>()}};

}  // namespace tg
