// pgq_k_sqwa_sel.hip -- kernel instantiations of the SQWA snapshot fold (MODE_SQWA):
// the percentile-select variant.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_sqwa_sel(bool table) { return kernel_ptr<MODE_SQWA, F_F32 | F_PASS | F_SEL>(table); }

}  // namespace pgq
