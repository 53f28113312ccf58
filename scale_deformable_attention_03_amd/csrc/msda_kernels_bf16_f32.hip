// The mixed-precision kernels (bf16 values, f32 per-sample tensors): explicit
// instantiation of their launches (a translation unit of its own, compiled in
// parallel with the others).
#include "msda_launch_impl.hpp"

template struct msda_host::Launch<msda::kBF16M>;
