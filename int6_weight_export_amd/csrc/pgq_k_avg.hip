// pgq_k_avg.hip -- kernel instantiations of weight averaging (EMA, SWA), the whole-tensor select
// (candidate pass and radix passes) and the grouped decode.
#include "pgq_kern.h"

namespace pgq {

const void* kernels_avg(int mode, uint32_t v, bool table)
{
    switch (mode) {
    case MODE_EMA: return average_kernel<MODE_EMA>(v, table);
    case MODE_TSEL: return average_kernel<MODE_TSEL>(v, table);
    case MODE_TCAND: return average_kernel<MODE_TCAND>(v, table);
    case MODE_SWA: return average_kernel<MODE_SWA>(v, table);
    case MODE_DECODE: return table ? reinterpret_cast<const void*>(&pgq_table_kernel<MODE_DECODE, F_F32>) : nullptr;
    default: return nullptr;
    }
}

}  // namespace pgq
