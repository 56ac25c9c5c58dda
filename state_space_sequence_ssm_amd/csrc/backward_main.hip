// The backward kernel's sequence-split main launch (the two segments' backward
// walks), a translation unit of its own so
// that the build runs in parallel.
#include "backward_impl.hpp"

namespace m3 {

hipError_t launch_backward_main(const BackwardParams& p, hipStream_t s) { return bw::launch_mode<2>(p, s); }

}  // namespace m3
