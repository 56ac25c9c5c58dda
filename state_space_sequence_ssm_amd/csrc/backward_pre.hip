// The backward kernel's sequence-split pre launch (segment 0's forward walk and
// segment 1's gradient sum), a translation unit of its own so
// that the build runs in parallel.
#include "backward_impl.hpp"

namespace m3 {

hipError_t launch_backward_pre(const BackwardParams& p, hipStream_t s) { return bw::launch_mode<1>(p, s); }

}  // namespace m3
