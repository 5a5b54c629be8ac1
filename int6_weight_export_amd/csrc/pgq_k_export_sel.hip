// pgq_k_export_sel.hip -- kernel instantiations of the whole-model export (int8 codes) (MODE_EXPORT):
// the percentile-select variant.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_export_sel(bool table) { return kernel_ptr<MODE_EXPORT, F_F32 | F_PASS | F_SEL>(table); }

}  // namespace pgq
