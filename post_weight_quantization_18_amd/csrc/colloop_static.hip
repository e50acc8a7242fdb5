// Column loop instantiated for static groups (see colloop_impl.h).
#include "colloop_impl.h"

namespace gptq {
template gptq_status_t launch_colloop<-2, false>(const ColArgs& a, hipStream_t st);
template gptq_status_t launch_colloop<-2, true>(const ColArgs& a, hipStream_t st);
}  // namespace gptq
