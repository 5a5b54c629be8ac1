// pgq_k_export_alls.hip -- kernel instantiations of the whole-model export (int8 codes) (MODE_EXPORT):
// every feature, single-matrix launches.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_export_all_single() { return kernel_ptr<MODE_EXPORT, F_ALL>(false); }

}  // namespace pgq
