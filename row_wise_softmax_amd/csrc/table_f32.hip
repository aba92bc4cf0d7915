// table_f32.hip -- the f32 instantiations of the kernel table (one translation
// unit per element type so the three compile in parallel).
#include "row_wise_softmax.h"
#include "kernel_table.hpp"
#include "softmax_kernels.hpp"

#define ELEM rws::F32
#define ELEM_NAME "f32"
#define ELEM_BYTES 4
#define DTYPE_CODE SOFTMAX_F32

namespace rws {

const Entry kTableF32[] = {
#include "table_entries.inc"
};
const int kTableF32Size = sizeof(kTableF32) / sizeof(kTableF32[0]);

}  // namespace rws
