// pgq_k_export6_sel.hip -- kernel instantiations of the export with 6-bit code storage (MODE_EXPORT6):
// the percentile-select variant.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_export6_sel(bool table) { return kernel_ptr<MODE_EXPORT6, F_F32 | F_PASS | F_SEL>(table); }

}  // namespace pgq
