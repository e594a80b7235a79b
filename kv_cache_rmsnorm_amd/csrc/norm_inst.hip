// norm_inst.hip -- one instantiation of the row-norm engine. The build
// compiles this file once per (KCR_NORM_T, KCR_NORM_ADD) pair, T in {Bf16,
// F16, F32}, so the six variants compile in parallel.
#include "norm_engine.h"

#if !defined(KCR_NORM_T) || !defined(KCR_NORM_ADD)
#error "compile with -DKCR_NORM_T=<Bf16|F16|F32> -DKCR_NORM_ADD=<0|1>"
#endif

namespace kcr {
template int run_norm<KCR_NORM_T, (KCR_NORM_ADD != 0)>(const NormArgs& a, void* stream);
}  // namespace kcr
