// Column loop instantiated for groups that start at block starts (cut blocks) (see colloop_impl.h).
#include "colloop_impl.h"

namespace gptq {
template gptq_status_t launch_colloop<-1, false>(const ColArgs& a, hipStream_t st);
}  // namespace gptq
