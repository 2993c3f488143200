// gemm_skinny_w.hip -- the few-row matrix-core kernel (gemm_skinny.h) for
// 2-, 3- and 8-bit weights.
#include "gemm_skinny.h"

namespace qmm {

hipError_t launch_gemm_skinny_w(const MatArgs& a) {
  switch (a.bits) {
    case 2: return launch_skinny_x<2>(a);
    case 3: return launch_skinny_x<3>(a);
    default: return launch_skinny_x<8>(a);
  }
}

}  // namespace qmm
