// unfused.hip -- the unfused five-operation softmax, as a measured baseline.
//
// The same result computed the way "GPU Kernels - Implementing and
// optimizing Softmax" writes its naive version (section "Baseline & Triton
// Softmax kernel") and "Kernel Fusion" counts it (section "Where the time goes
// in an elementwise chain"): five separate kernels, each a round trip through
// HBM --
//   1. m   = rowmax(x)          reads x
//   2. z   = x - m              reads x, writes z
//   3. num = exp(z)             reads z, writes num
//   4. s   = rowsum(num)        reads num
//   5. y   = num / s            reads num, writes y
// -- five reads and three writes of the tensor, 4x the traffic of the fused
// kernels.  z and num are held in the element type (as separate framework ops
// would), m and s in fp32.  Each kernel is written well (16-byte accesses, one
// workgroup per row with a wave64 + LDS reduction for the two reductions);
// only the fusion is missing.  Measurement only: rows must be 16-byte aligned
// and rows with no finite entry give NaN, as the five separate ops do.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "row_wise_softmax.h"
#include "softmax_kernels.hpp"

namespace {

using rws::Access;
using rws::kWave;

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int64_t kMaxGrid = int64_t(1) << 20;

struct UArgs {
    const void* src;   // input of this op
    void* dst;         // output of this op (tensor ops)
    const float* vec;  // per-row operand (sub, div)
    float* red;        // per-row result (max, sum)
    int64_t rows;
    int64_t src_stride;  // accesses
    int64_t dst_stride;  // accesses
    int nacc;
};

enum class Red { Max, Sum };
enum class Ew { Sub, Exp, Div };

template <Red R>
__device__ inline float red_op(float a, float b) {
    if constexpr (R == Red::Max) return fmaxf(a, b);
    else return a + b;
}

// One workgroup per row: a row reduction (max or sum) written to red[row].
template <class E, Red R>
__global__ void __launch_bounds__(kThreads) unfused_reduce(UArgs a) {
    typedef typename Access<E, 16 / E::kBytes>::raw raw;
    constexpr int N = 16 / E::kBytes;
    __shared__ float part[kWaves];
    const raw* src = static_cast<const raw*>(a.src);
    const int t = threadIdx.x;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        float acc = R == Red::Max ? -INFINITY : 0.0f;
        for (int i = t; i < a.nacc; i += kThreads) {
            float f[N];
            rws::load_elems<E, N>(src + row * a.src_stride + i, f);
#pragma unroll
            for (int e = 0; e < N; ++e) acc = red_op<R>(acc, f[e]);
        }
        if constexpr (R == Red::Max) acc = rws::group_reduce<kWave, rws::OpMax>(acc);
        else acc = rws::group_reduce<kWave, rws::OpSum>(acc);
        if ((t & (kWave - 1)) == 0) part[t / kWave] = acc;
        __syncthreads();
        if (t == 0) {
            float r = part[0];
#pragma unroll
            for (int w = 1; w < kWaves; ++w) r = red_op<R>(r, part[w]);
            a.red[row] = r;
        }
        __syncthreads();  // part[] is rewritten for the next row
    }
}

// One workgroup per row: an elementwise op with an optional per-row operand.
template <class E, Ew OP>
__global__ void __launch_bounds__(kThreads) unfused_elementwise(UArgs a) {
    typedef typename Access<E, 16 / E::kBytes>::raw raw;
    constexpr int N = 16 / E::kBytes;
    const raw* src = static_cast<const raw*>(a.src);
    raw* dst = static_cast<raw*>(a.dst);
    const int t = threadIdx.x;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const float v = OP == Ew::Exp ? 0.0f : a.vec[row];
        for (int i = t; i < a.nacc; i += kThreads) {
            float f[N];
            rws::load_elems<E, N>(src + row * a.src_stride + i, f);
#pragma unroll
            for (int e = 0; e < N; ++e) {
                if constexpr (OP == Ew::Sub) f[e] = f[e] - v;
                else if constexpr (OP == Ew::Exp) f[e] = __builtin_amdgcn_exp2f(f[e] * rws::kLog2e);
                else f[e] = f[e] / v;
            }
            rws::store_elems<E, N>(dst + row * a.dst_stride + i, f);
        }
    }
}

int elem_bytes(int dtype) { return dtype == SOFTMAX_F32 ? 4 : 2; }

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Workspace layout: z (rows x cols, dense), num (rows x cols, dense), m (rows
// floats), s (rows floats), each part 256-byte aligned.
int64_t workspace_bytes(int64_t rows, int64_t cols, int dtype) {
    const int64_t t = round_up(rows * cols * elem_bytes(dtype), 256);
    const int64_t v = round_up(rows * 4, 256);
    return 2 * t + 2 * v;
}

template <class E>
int run5(const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride, char* ws, hipStream_t stream) {
    constexpr int N = 16 / E::kBytes;
    const int64_t t = round_up(rows * cols * E::kBytes, 256);
    const int64_t v = round_up(rows * 4, 256);
    void* z = ws;
    void* num = ws + t;
    float* m = reinterpret_cast<float*>(ws + 2 * t);
    float* s = reinterpret_cast<float*>(ws + 2 * t + v);
    const int64_t io = row_stride / N, dense = cols / N;
    const int nacc = int(cols / N);
    const dim3 grid(unsigned(rows < kMaxGrid ? rows : kMaxGrid)), block(kThreads);
    UArgs a[5] = {
        {in, nullptr, nullptr, m, rows, io, 0, nacc},       // m = max x
        {in, z, m, nullptr, rows, io, dense, nacc},         // z = x - m
        {z, num, nullptr, nullptr, rows, dense, dense, nacc},  // num = exp z
        {num, nullptr, nullptr, s, rows, dense, 0, nacc},   // s = sum num
        {num, out, s, nullptr, rows, dense, io, nacc},      // y = num / s
    };
    const void* fns[5] = {
        (const void*)&unfused_reduce<E, Red::Max>, (const void*)&unfused_elementwise<E, Ew::Sub>,
        (const void*)&unfused_elementwise<E, Ew::Exp>, (const void*)&unfused_reduce<E, Red::Sum>,
        (const void*)&unfused_elementwise<E, Ew::Div>,
    };
    for (int k = 0; k < 5; ++k) {
        void* args[] = {&a[k]};
        if (hipLaunchKernel(fns[k], grid, block, args, 0, stream) != hipSuccess) {
            (void)hipGetLastError();
            return SOFTMAX_ERR_HIP;
        }
    }
    return SOFTMAX_OK;
}

}  // namespace

extern "C" {

int64_t softmax_unfused_workspace_bytes(int64_t rows, int64_t cols, int dtype) {
    if (rows < 0 || cols < 0 || (dtype != SOFTMAX_F32 && dtype != SOFTMAX_F16 && dtype != SOFTMAX_BF16)) return -1;
    if (rows > 0 && cols > (INT64_MAX / 4 - 1024) / rows / 2) return -1;
    return workspace_bytes(rows, cols, dtype);
}

int softmax_unfused_5op(const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
                        void* workspace, int64_t workspace_size, void* stream) {
    if (dtype != SOFTMAX_F32 && dtype != SOFTMAX_F16 && dtype != SOFTMAX_BF16) return SOFTMAX_ERR_BAD_DTYPE;
    if (rows < 0 || cols < 0) return SOFTMAX_ERR_BAD_SHAPE;
    if (rows == 0 || cols == 0) return SOFTMAX_OK;
    if (in == nullptr || out == nullptr || workspace == nullptr) return SOFTMAX_ERR_NULL_POINTER;
    const int64_t esz = elem_bytes(dtype);
    if (row_stride < cols || cols > (int64_t(1) << 30)) return SOFTMAX_ERR_BAD_SHAPE;
    if (rows - 1 > (INT64_MAX / esz - cols) / row_stride) return SOFTMAX_ERR_BAD_SHAPE;
    if (uintptr_t(in) % 16 || uintptr_t(out) % 16 || uintptr_t(workspace) % 256 || (row_stride * esz) % 16 ||
        (cols * esz) % 16)
        return SOFTMAX_ERR_BAD_SHAPE;
    const int64_t need = softmax_unfused_workspace_bytes(rows, cols, dtype);
    if (need < 0 || workspace_size < need) return SOFTMAX_ERR_BAD_SHAPE;
    const int64_t extent = ((rows - 1) * row_stride + cols) * esz;
    const uintptr_t a = uintptr_t(in), b = uintptr_t(out), w = uintptr_t(workspace);
    if (a != b && a < b + uint64_t(extent) && b < a + uint64_t(extent)) return SOFTMAX_ERR_OVERLAP;
    if ((w < a + uint64_t(extent) && a < w + uint64_t(need)) || (w < b + uint64_t(extent) && b < w + uint64_t(need)))
        return SOFTMAX_ERR_OVERLAP;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    switch (dtype) {
        case SOFTMAX_F32: return run5<rws::F32>(in, out, rows, cols, row_stride, ws, st);
        case SOFTMAX_F16: return run5<rws::F16>(in, out, rows, cols, row_stride, ws, st);
        default: return run5<rws::BF16>(in, out, rows, cols, row_stride, ws, st);
    }
}

}  // extern "C"
