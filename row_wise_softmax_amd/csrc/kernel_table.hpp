// kernel_table.hpp -- the compiled table of kernel instantiations.
//
// Each entry is one template instantiation of a kernel in softmax_kernels.hpp
// with its launch parameters.  softmax_fwd picks an entry by width; the bench
// and the tests can force any entry (softmax_fwd_kernel) to sweep block shapes
// per width, in the spirit of measuring threads-per-block candidates per shape
// and keeping the winner ("GPU Kernels - Implementing and optimizing Softmax",
// section "Autotuning") -- done offline here, with the winners compiled into
// the dispatch rule, so no call ever times anything.
#pragma once

#include <stdint.h>

namespace rws {

struct Entry {
    int dtype;    // SOFTMAX_F32 / F16 / BF16
    int variant;  // SOFTMAX_VARIANT_*
    bool causal;  // scaled, causally masked softmax (softmax_fwd_causal)
    bool any;     // 16-byte accesses for rows at any element offset (in and out at one offset mod 16)
    int vec;      // elements per access
    int lanes;    // packed: lanes per row; row/online: threads per row
    int vpl;      // accesses per lane per row (online: per chunk)
    int groups;   // packed: row groups per wave; else 1
    int block;    // threads per workgroup (packed: maximum)
    const void* fn;
    const void* fn_shifted;  // row kernels: the line-shifted instantiation; else null
    const char* name;
};

extern const Entry kTableF32[];
extern const int kTableF32Size;
extern const Entry kTableF16[];
extern const int kTableF16Size;
extern const Entry kTableBF16[];
extern const int kTableBF16Size;

}  // namespace rws
