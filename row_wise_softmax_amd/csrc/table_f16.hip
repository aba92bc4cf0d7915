// table_f16.hip -- the f16 instantiations of the kernel table (one translation
// unit per element type so the three compile in parallel).
#include "row_wise_softmax.h"
#include "kernel_table.hpp"
#include "softmax_kernels.hpp"

#define ELEM rws::F16
#define ELEM_NAME "f16"
#define ELEM_BYTES 2
#define DTYPE_CODE SOFTMAX_F16

namespace rws {

const Entry kTableF16[] = {
#include "table_entries.inc"
};
const int kTableF16Size = sizeof(kTableF16) / sizeof(kTableF16[0]);

}  // namespace rws
