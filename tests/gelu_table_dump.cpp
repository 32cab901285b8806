// Prints the GELU table that the HIP library builds at compile time
// (csrc/gelu_table.h), one hexadecimal entry per line, for its CPU test.
#include <cstdio>

#include "../bit_w4a4_quantized_svdq_amd/csrc/gelu_table.h"

int main() {
    constexpr auto tab = svdq::make_gelu_table();   // evaluated by the compiler, as in the library
    std::printf("%d %d %d\n", svdq::GELU_E_LO, svdq::GELU_STRIDE, svdq::GELU_TAB);
    for (int i = 0; i < svdq::GELU_TAB_PAD; ++i) std::printf("%04x\n", tab[i]);
    return 0;
}
