// pgq_k_export_allt.hip -- kernel instantiations of the whole-model export (int8 codes) (MODE_EXPORT):
// every feature, grouped launches.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_export_all_table() { return kernel_ptr<MODE_EXPORT, F_ALL>(true); }

}  // namespace pgq
