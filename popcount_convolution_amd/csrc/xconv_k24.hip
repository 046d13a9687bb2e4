// Compiled instances of the specialised XNOR / AND convolution kernel for
// 2x2 and 4x4 windows (the centred window of an even kernel pads k/2
// before and k/2 - 1 after): (KH, KW, words per pixel, horizontal stride) at each strip width.
#include "xconv_fast.h"

namespace bconv {
namespace {

const FastEntry kTable[] = {
    BCONV_FAST_P(2, 2, 1, 1), BCONV_FAST_P(2, 2, 2, 1), BCONV_FAST_P(2, 2, 4, 1),
    BCONV_FAST_P(4, 4, 1, 1), BCONV_FAST_P(4, 4, 2, 1), BCONV_FAST_P(4, 4, 4, 1),
    // stride 2
    BCONV_FAST_P(2, 2, 1, 2), BCONV_FAST_P(2, 2, 2, 2), BCONV_FAST_P(2, 2, 4, 2),
    BCONV_FAST_P(4, 4, 1, 2), BCONV_FAST_P(4, 4, 2, 2), BCONV_FAST_P(4, 4, 4, 2),
};

}  // namespace

FastTable xconv_fast_k24() { return {kTable, (int)(sizeof(kTable) / sizeof(kTable[0]))}; }

}  // namespace bconv
