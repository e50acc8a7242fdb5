// Column loop instantiated for one grid per row (see colloop_impl.h).
#include "colloop_impl.h"

namespace gptq {
template gptq_status_t launch_colloop<0, false>(const ColArgs& a, hipStream_t st);
template gptq_status_t launch_colloop<0, true>(const ColArgs& a, hipStream_t st);
}  // namespace gptq
