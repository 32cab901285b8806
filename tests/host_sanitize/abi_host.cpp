// The C ABI layer of libsvdq (its host-side argument checks and dispatch),
// compiled for the host alone so that AddressSanitizer and
// UndefinedBehaviorSanitizer can watch it.  The kernels' launchers and the
// three HIP runtime calls the layer makes come from hip_stubs.cpp.
#include "../../bit_w4a4_quantized_svdq_amd/csrc/svdq_abi.hip"
