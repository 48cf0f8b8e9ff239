// Scoring kernels for the C_BF16Q_FP8K operand combination (see score_kernels.h).
#include "score_kernels.h"

namespace dosa {

hipError_t launch_score_bf16fp8(int H, int d, const ScoreLaunch& p, hipStream_t s) {
  return launch_score_c<C_BF16Q_FP8K>(H, d, p, s);
}

}  // namespace dosa
