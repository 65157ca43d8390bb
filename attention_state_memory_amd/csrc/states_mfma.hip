// Prefix attention states on MFMA (bf16).  Placeholder dispatch: every shape
// currently runs the plain VALU kernel.
#include "common.hpp"
#include "kernels.hpp"

namespace asmk {

bool states_fast_path(int dtype, int d, int G) {
  (void)dtype; (void)d; (void)G;
  return false;
}

hipError_t launch_build_states(const StatesArgs& a, int dtype, hipStream_t s) {
  return launch_states_generic(a, dtype, s);
}

}  // namespace asmk
