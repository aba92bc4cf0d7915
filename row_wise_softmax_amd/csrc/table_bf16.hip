// table_bf16.hip -- the bf16 instantiations of the kernel table (one translation
// unit per element type so the three compile in parallel).
#include "row_wise_softmax.h"
#include "kernel_table.hpp"
#include "softmax_kernels.hpp"

#define ELEM rws::BF16
#define ELEM_NAME "bf16"
#define ELEM_BYTES 2
#define DTYPE_CODE SOFTMAX_BF16

namespace rws {

const Entry kTableBF16[] = {
#include "table_entries.inc"
};
const int kTableBF16Size = sizeof(kTableBF16) / sizeof(kTableBF16[0]);

}  // namespace rws
