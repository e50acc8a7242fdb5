// Column loop instantiated for groups of 64 (see colloop_impl.h).
#include "colloop_impl.h"

namespace gptq {
template gptq_status_t launch_colloop<64, false>(const ColArgs& a, hipStream_t st);
template gptq_status_t launch_colloop<64, true>(const ColArgs& a, hipStream_t st);
}  // namespace gptq
