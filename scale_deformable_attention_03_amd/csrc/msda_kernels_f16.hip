// The f16 kernels of the library: explicit instantiation of their launches
// (a translation unit of its own, compiled in parallel with the others).
#include "msda_launch_impl.hpp"

template struct msda_host::Launch<msda_host::kF16>;
