// Tile-study kernels in the other output modes of the deviation study (page
// "Is Flash Attention Stable?" explainer, aibr.jp, sections 3 and 4): O
// written in fp32 before its final rounding, and the running output held in
// bf16 between key tiles.  Every (Br, Bc) in {16, 32, 64, 128}^2 for d = 64
// and 128.  The kernel is in fa_study_kernel.h.
#include "fa_study_kernel.h"

namespace fa {
namespace {

#define FA_MODE(D, BR, BC, CAUSAL, MODE)                                               \
    Instance {                                                                         \
        D, CAUSAL, BR, BC,                                                             \
            &launch_bf16<D, BC, Pick<BR, BC>::MF, Pick<BR, BC>::NW, CAUSAL, MODE>      \
    }
#define FA_MODE_BOTH(D, BR, BC, MODE) FA_MODE(D, BR, BC, false, MODE), FA_MODE(D, BR, BC, true, MODE)
#define FA_MODE_ROW(D, BR, MODE) \
    FA_MODE_BOTH(D, BR, 16, MODE), FA_MODE_BOTH(D, BR, 32, MODE), FA_MODE_BOTH(D, BR, 64, MODE), \
        FA_MODE_BOTH(D, BR, 128, MODE)
#define FA_MODE_TABLE(MODE)                                                            \
    FA_MODE_ROW(128, 16, MODE), FA_MODE_ROW(128, 32, MODE), FA_MODE_ROW(128, 64, MODE), \
        FA_MODE_ROW(128, 128, MODE), FA_MODE_ROW(64, 16, MODE), FA_MODE_ROW(64, 32, MODE), \
        FA_MODE_ROW(64, 64, MODE), FA_MODE_ROW(64, 128, MODE)

}  // namespace

const Instance *bf16_f32out_instances() {
    static const Instance table[] = {FA_MODE_TABLE(kModeF32Out), Instance{0, 0, 0, 0, nullptr}};
    return table;
}

const Instance *bf16_acc16_instances() {
    static const Instance table[] = {FA_MODE_TABLE(kModeAcc16), Instance{0, 0, 0, 0, nullptr}};
    return table;
}

}  // namespace fa
