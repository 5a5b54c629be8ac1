// pgq_k_export6.hip -- kernel instantiations of the export with 6-bit code storage (MODE_EXPORT6):
// the lean streaming variants.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_export6(uint32_t v, bool table) { return export_like_lean<MODE_EXPORT6>(v, table); }

}  // namespace pgq
