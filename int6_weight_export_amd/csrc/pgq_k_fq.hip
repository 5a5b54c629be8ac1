// pgq_k_fq.hip -- kernel instantiations of STE fake quantization (forward(+backward), backward).
#include "pgq_kern.h"

namespace pgq {

const void* kernels_fq(int mode, uint32_t v, bool table)
{
    if (mode == MODE_FQ_BWD) return kernel_ptr<MODE_FQ_BWD, F_ALL>(table);
    if (v == F_BF16) return kernel_ptr<MODE_FQ, F_BF16>(table);
    if (v == (F_BF16 | F_SEL)) return kernel_ptr<MODE_FQ, F_BF16 | F_SEL>(table);
    return kernel_ptr<MODE_FQ, F_ALL>(table);
}

}  // namespace pgq
