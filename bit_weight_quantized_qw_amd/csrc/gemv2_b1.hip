// Instantiations of the 2-bit decode GEMV for batch width 1.
#include "gemv2_kernel.h"

namespace qw {
namespace gemv2 {

qw_status launch_b1(const Args &a, int UW, int UA, int grid, int threads, size_t lds,
                     hipStream_t s) {
  switch (UW) {
      case 1: return launch_ua<1, 1>(a, UA, grid, threads, lds, s);
      case 2: return launch_ua<1, 2>(a, UA, grid, threads, lds, s);
      case 3: return launch_ua<1, 3>(a, UA, grid, threads, lds, s);
      case 4: return launch_ua<1, 4>(a, UA, grid, threads, lds, s);
      case 5: return launch_ua<1, 5>(a, UA, grid, threads, lds, s);
      case 6: return launch_ua<1, 6>(a, UA, grid, threads, lds, s);
      case 7: return launch_ua<1, 7>(a, UA, grid, threads, lds, s);
      default: return launch_ua<1, 8>(a, UA, grid, threads, lds, s);
  }
}

}  // namespace gemv2
}  // namespace qw
