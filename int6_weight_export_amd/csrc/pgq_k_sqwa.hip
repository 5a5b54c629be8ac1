// pgq_k_sqwa.hip -- kernel instantiations of the SQWA snapshot fold (MODE_SQWA):
// the lean streaming variants.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_sqwa(uint32_t v, bool table) { return export_like_lean<MODE_SQWA>(v, table); }

}  // namespace pgq
