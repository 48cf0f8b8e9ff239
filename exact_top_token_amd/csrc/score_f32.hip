// Scoring kernels for the C_F32 operand combination (see score_kernels.h).
#include "score_kernels.h"

namespace dosa {

hipError_t launch_score_f32(int H, int d, const ScoreLaunch& p, hipStream_t s) {
  return launch_score_c<C_F32>(H, d, p, s);
}

}  // namespace dosa
