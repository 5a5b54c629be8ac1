// pgq_k_sqwa_allt.hip -- kernel instantiations of the SQWA snapshot fold (MODE_SQWA):
// every feature, grouped launches.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_sqwa_all_table() { return kernel_ptr<MODE_SQWA, F_ALL>(true); }

}  // namespace pgq
