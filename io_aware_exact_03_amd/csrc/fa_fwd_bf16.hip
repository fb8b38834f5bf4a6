// Tile-study kernels with bf16 output: every (Br, Bc) in {16, 32, 64, 128}^2
// for d = 64 and 128 (the tile-size axis of the deviation study on the page
// "Is Flash Attention Stable?" explainer, aibr.jp, sections 3 and 4).  The
// kernel itself is in fa_study_kernel.h.
#include "fa_study_kernel.h"

namespace fa {
namespace {

#define FA_BF16(D, BR, BC, CAUSAL)                                             \
    Instance {                                                                 \
        D, CAUSAL, BR, BC,                                                     \
            &launch_bf16<D, BC, Pick<BR, BC>::MF, Pick<BR, BC>::NW, CAUSAL>    \
    }
#define FA_BF16_BOTH(D, BR, BC) FA_BF16(D, BR, BC, false), FA_BF16(D, BR, BC, true)
#define FA_BF16_ROW(D, BR) \
    FA_BF16_BOTH(D, BR, 16), FA_BF16_BOTH(D, BR, 32), FA_BF16_BOTH(D, BR, 64), FA_BF16_BOTH(D, BR, 128)


}  // namespace

const Instance *bf16_instances() {
    // Tile-size study: every (Br, Bc) in {16, 32, 64, 128}^2 for d = 64 and 128.
    static const Instance table[] = {
        FA_BF16_ROW(128, 16),
        FA_BF16_ROW(128, 32),
        FA_BF16_ROW(128, 64),
        FA_BF16_ROW(128, 128),
        FA_BF16_ROW(64, 16),
        FA_BF16_ROW(64, 32),
        FA_BF16_ROW(64, 64),
        FA_BF16_ROW(64, 128),
        Instance{0, 0, 0, 0, nullptr},
    };
    return table;
}

}  // namespace fa
