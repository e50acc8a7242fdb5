// Column loop instantiated for groups of 16 (see colloop_impl.h).
#include "colloop_impl.h"

namespace gptq {
template gptq_status_t launch_colloop<16, false>(const ColArgs& a, hipStream_t st);
template gptq_status_t launch_colloop<16, true>(const ColArgs& a, hipStream_t st);
}  // namespace gptq
