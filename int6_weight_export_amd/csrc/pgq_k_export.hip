// pgq_k_export.hip -- kernel instantiations of the whole-model export (int8 codes) (MODE_EXPORT):
// the lean streaming variants.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_export(uint32_t v, bool table) { return export_like_lean<MODE_EXPORT>(v, table); }

}  // namespace pgq
