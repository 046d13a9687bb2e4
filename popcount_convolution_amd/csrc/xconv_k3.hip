// Compiled instances of the specialised XNOR / AND convolution kernel for
// 3x3 windows: (KH, KW, words per pixel, horizontal stride) at each strip width.
#include "xconv_fast.h"

namespace bconv {
namespace {

const FastEntry kTable[] = {
    BCONV_FAST_P(3, 3, 1, 1), BCONV_FAST_P(3, 3, 2, 1), BCONV_FAST_P(3, 3, 3, 1),
    BCONV_FAST_P(3, 3, 4, 1), BCONV_FAST_P(3, 3, 8, 1),
    // stride 2
    BCONV_FAST_P(3, 3, 1, 2), BCONV_FAST_P(3, 3, 2, 2), BCONV_FAST_P(3, 3, 4, 2),
    BCONV_FAST_P(3, 3, 8, 2),
};

}  // namespace

FastTable xconv_fast_k3() { return {kTable, (int)(sizeof(kTable) / sizeof(kTable[0]))}; }

}  // namespace bconv
