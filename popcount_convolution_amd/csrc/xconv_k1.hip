// Compiled instances of the specialised XNOR / AND convolution kernel for
// 1x1 windows: (KH, KW, words per pixel, horizontal stride) at each strip width.
#include "xconv_fast.h"

namespace bconv {
namespace {

const FastEntry kTable[] = {
    BCONV_FAST_P(1, 1, 1, 1), BCONV_FAST_P(1, 1, 2, 1), BCONV_FAST_P(1, 1, 4, 1), BCONV_FAST_P(1, 1, 8, 1),
    // stride 2
    BCONV_FAST_P(1, 1, 1, 2), BCONV_FAST_P(1, 1, 2, 2), BCONV_FAST_P(1, 1, 4, 2), BCONV_FAST_P(1, 1, 8, 2),
};

}  // namespace

FastTable xconv_fast_k1() { return {kTable, (int)(sizeof(kTable) / sizeof(kTable[0]))}; }

}  // namespace bconv
