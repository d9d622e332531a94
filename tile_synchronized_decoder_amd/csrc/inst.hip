// One instantiation of the decoder kernels: element type MK_WT (bf16 bits or
// float) and batch bucket MK_NB.  The build compiles this file once per
// (type, bucket) pair, in parallel, and links the tables together.
#include "kernels.h"

#ifndef MK_WT
#error "define MK_WT (uint16_t or float) and MK_NB"
#endif

#define MK_CAT2(a, b, c) a##b##_##c
#define MK_CAT(a, b, c) MK_CAT2(a, b, c)

namespace mkd {
Table MK_CAT(table_, MK_WT_NAME, MK_NB)() {
  using LT = Launch<MK_WT, MK_NB>;
  return {LT::prep, LT::mega, LT::kHasLoop ? LT::loop : nullptr, LT::kpo, LT::ms, LT::prep_lm, LT::lm};
}
}  // namespace mkd
