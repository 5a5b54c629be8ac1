// pgq_k_sqwa_alls.hip -- kernel instantiations of the SQWA snapshot fold (MODE_SQWA):
// every feature, single-matrix launches.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_sqwa_all_single() { return kernel_ptr<MODE_SQWA, F_ALL>(false); }

}  // namespace pgq
