// pgq_k_export6_allt.hip -- kernel instantiations of the export with 6-bit code storage (MODE_EXPORT6):
// every feature, grouped launches.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_export6_all_table() { return kernel_ptr<MODE_EXPORT6, F_ALL>(true); }

}  // namespace pgq
