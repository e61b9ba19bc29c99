// Instantiations of the 2-bit decode GEMV for batch width 2.
#include "gemv2_kernel.h"

namespace qw {
namespace gemv2 {

qw_status launch_b2(const Args &a, int UW, int UA, int grid, int threads, size_t lds,
                     hipStream_t s) {
  switch (UW) {
      case 1: return launch_ua<2, 1>(a, UA, grid, threads, lds, s);
      case 2: return launch_ua<2, 2>(a, UA, grid, threads, lds, s);
      default: return launch_ua<2, 3>(a, UA, grid, threads, lds, s);
  }
}

}  // namespace gemv2
}  // namespace qw
