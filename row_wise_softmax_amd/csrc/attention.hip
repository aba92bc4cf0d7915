// attention.hip -- fused attention forward O = softmax(scale Q K^T) V on MFMA.
//
// The softmax of this library inside the attention it usually serves: scores
// Q K^T scaled by `scale` (1/sqrt(d) in "Dissecting Memory Bandwidth & SRAM
// Tiling in Triton", section "Memory Hierarchy: Why Standard Attention
// Collapses"), an optional causal mask, the row softmax, and the product with
// V, fused so the nq x nk score matrix never reaches HBM.  The softmax runs
// online over key blocks: running row max m and normaliser l, with the output
// accumulator rescaled whenever the max grows (same page, section "The
// Mathematical Remedy: Online Softmax Tiling", and the kernel of section
// "Writing the Kernel in OpenAI Triton").  This is a contraction, so both
// products run on the matrix cores: v_mfma_f32_16x16x32_{f16,bf16}.
//
// Work split: one workgroup of 4 waves per (batch*head, block of 64 queries);
// each wave owns 16 query rows and keeps their Q fragments in registers.  Per
// block of 64 keys the workgroup stages K (row-major) and V (transposed) in
// LDS; each wave computes its 16 x 64 score tile with MFMA, updates m and l
// in fp32 (exponentials as 2^(x log2 e) on v_exp_f32), writes P in the input
// type to a wave-private LDS tile, reads it back in the MFMA A-operand layout
// and accumulates O += P V.
//
// MFMA operand layout used (16 x 16 x 32): lane L supplies row (or column)
// L % 16 and eight consecutive k slots 8 (L / 16) .. 8 (L / 16) + 7; the
// 16 x 16 fp32 result lands with column L % 16 and rows 4 (L / 16) .. + 3 in
// the lane's four accumulators.  Both operands of every product are filled
// with the same slot -> k assignment, so the sum over k is the same whatever
// order the hardware walks the slots in.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "row_wise_softmax.h"
#include "softmax_kernels.hpp"

namespace {

using rws::kWave;
using rws::u32x4;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 64;  // queries per workgroup (16 per wave)
constexpr int kBN = 64;  // keys per block
constexpr int kThreads = 256;
constexpr double kLog2eD = 1.4426950408889634074;

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int64_t nq;
    int64_t nk;
    int64_t offset;  // causal: query i keeps keys j <= i + offset (offset = nk - nq)
    float coef;      // scale * log2(e)
};

template <class E>
__device__ inline f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    if constexpr (std::is_same_v<E, rws::F16>)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ inline u32x4 lds16(const unsigned short* p) { return *reinterpret_cast<const u32x4*>(p); }

template <class E, int D, bool Causal>
__global__ void __launch_bounds__(kThreads) attention_fwd_kernel(AttnArgs a) {
    constexpr int kKS = D / 32;      // MFMA k-steps over the head dimension
    constexpr int kKP = D + 8;       // padded K row in LDS (halves)
    constexpr int kVP = kBN + 8;     // padded V^T row (keys)
    constexpr int kPP = kBN + 8;     // padded P row (keys)
    constexpr int kDT = D / 16;      // 16-wide output tiles per wave
    __shared__ __attribute__((aligned(16))) unsigned short sK[kBN * kKP];
    __shared__ __attribute__((aligned(16))) unsigned short sVt[D * kVP];
    __shared__ __attribute__((aligned(16))) unsigned short sP[4][16 * kPP];

    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int w = t / kWave;
    const int g = lane >> 4;  // lane group: k slots 8g .. 8g + 7, result rows 4g .. 4g + 3
    const int c = lane & 15;  // operand row / column, result column
    const int64_t bh = blockIdx.y;
    const int64_t m0 = int64_t(blockIdx.x) * kBM;
    const unsigned short* qb = static_cast<const unsigned short*>(a.q) + bh * a.nq * D;
    const unsigned short* kb = static_cast<const unsigned short*>(a.k) + bh * a.nk * D;
    const unsigned short* vb = static_cast<const unsigned short*>(a.v) + bh * a.nk * D;
    unsigned short* ob = static_cast<unsigned short*>(a.o) + bh * a.nq * D;

    // Q fragments of this wave's 16 rows (A operand): row m0 + 16w + c.
    u32x4 qf[kKS];
    {
        const int64_t row = m0 + 16 * w + c;
#pragma unroll
        for (int s = 0; s < kKS; ++s) {
            if (row < a.nq) qf[s] = rws::ld<true>(reinterpret_cast<const u32x4*>(qb + row * D + 32 * s + 8 * g));
            else qf[s] = u32x4{0, 0, 0, 0};
        }
    }

    float mrow[4], lrow[4];
    f32x4 oacc[kDT];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        mrow[r] = -INFINITY;
        lrow[r] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kDT; ++u) oacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Keys any query of this block may see.
    int64_t kend = a.nk;
    if (Causal) {
        const int64_t last = m0 + kBM - 1 + a.offset + 1;
        kend = last < kend ? last : kend;
    }

    for (int64_t n0 = 0; n0 < kend; n0 += kBN) {
        __syncthreads();  // every wave is done with the previous block's sK / sVt
        // Stage K (row-major) and V (transposed) for keys n0 .. n0 + 63.
        for (int idx = t; idx < kBN * D / 8; idx += kThreads) {
            const int key = idx / (D / 8);
            const int dc = (idx % (D / 8)) * 8;
            u32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
            if (n0 + key < a.nk) {
                kv = rws::ld<false>(reinterpret_cast<const u32x4*>(kb + (n0 + key) * D + dc));
                vv = rws::ld<false>(reinterpret_cast<const u32x4*>(vb + (n0 + key) * D + dc));
            }
            *reinterpret_cast<u32x4*>(sK + key * kKP + dc) = kv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sVt[(dc + 2 * e) * kVP + key] = (unsigned short)(vv[e] & 0xffffu);
                sVt[(dc + 2 * e + 1) * kVP + key] = (unsigned short)(vv[e] >> 16);
            }
        }
        __syncthreads();

        // Scores of this wave's 16 rows against the 64 keys (four 16 x 16 tiles).
        f32x4 sacc[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < kKS; ++s) sacc[nt] = mfma<E>(qf[s], lds16(sK + (16 * nt + c) * kKP + 32 * s + 8 * g), sacc[nt]);
        }

        // Scale into the log2 domain, mask, and update the running statistics.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t qi = m0 + 16 * w + 4 * g + r;
            float bm = -INFINITY;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int64_t kj = n0 + 16 * nt + c;
                float x = sacc[nt][r] * a.coef;
                if (kj >= a.nk || (Causal && kj > qi + a.offset)) x = -INFINITY;
                sacc[nt][r] = x;
                bm = fmaxf(bm, x);
            }
            bm = rws::group_reduce<16, rws::OpMax>(bm);  // the 16 lanes holding this row
            const float mnew = fmaxf(mrow[r], bm);
            const float msafe = mnew == -INFINITY ? 0.0f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(mrow[r] - msafe);  // 0 while the row had nothing
            float ps = 0.0f;
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const float p = __builtin_amdgcn_exp2f(sacc[nt][r] - msafe);
                sacc[nt][r] = p;
                ps += p;
            }
            lrow[r] = lrow[r] * alpha + ps;  // per-lane partial; summed over the row's lanes at the end
            mrow[r] = mnew;
#pragma unroll
            for (int u = 0; u < kDT; ++u) oacc[u][r] *= alpha;
        }

        // P in the input type, to this wave's LDS tile (row-major).
        unsigned short* pw = sP[w];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float pv = sacc[nt][r];
                pw[(4 * g + r) * kPP + 16 * nt + c] = rws::narrow_half<E>(pv);
            }
        __syncthreads();  // P writes visible before the A-operand reads

        // O += P V over the block's 64 keys (two k-steps of 32).
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const u32x4 pa = lds16(pw + c * kPP + 32 * s + 8 * g);
#pragma unroll
            for (int u = 0; u < kDT; ++u)
                oacc[u] = mfma<E>(pa, lds16(sVt + (16 * u + c) * kVP + 32 * s + 8 * g), oacc[u]);
        }
    }

    // Normalise and store: result rows 4g + r, column 16u + c.
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float l = rws::group_reduce<16, rws::OpSum>(lrow[r]);
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        const int64_t qi = m0 + 16 * w + 4 * g + r;
        if (qi < a.nq) {
#pragma unroll
            for (int u = 0; u < kDT; ++u) ob[qi * D + 16 * u + c] = rws::narrow_half<E>(oacc[u][r] * inv);
        }
    }
}

template <class E>
const void* pick(int64_t d, bool causal) {
    if (d == 64) return causal ? (const void*)&attention_fwd_kernel<E, 64, true> : (const void*)&attention_fwd_kernel<E, 64, false>;
    return causal ? (const void*)&attention_fwd_kernel<E, 128, true> : (const void*)&attention_fwd_kernel<E, 128, false>;
}

}  // namespace

extern "C" int attention_fwd(const void* q, const void* k, const void* v, void* o, int64_t batch, int64_t heads,
                             int64_t nq, int64_t nk, int64_t head_dim, float scale, int causal, int dtype,
                             void* stream) {
    if (dtype != SOFTMAX_F16 && dtype != SOFTMAX_BF16) return SOFTMAX_ERR_BAD_DTYPE;
    if (batch < 0 || heads < 0 || nq < 0 || nk < 0) return SOFTMAX_ERR_BAD_SHAPE;
    if (head_dim != 64 && head_dim != 128) return SOFTMAX_ERR_BAD_SHAPE;
    if (!(scale > 0.0f) || isinf(scale) || !(double(scale) * kLog2eD <= 3.0e38)) return SOFTMAX_ERR_BAD_SCALE;
    if (causal != 0 && causal != 1) return SOFTMAX_ERR_BAD_SHAPE;
    if (batch == 0 || heads == 0 || nq == 0) return SOFTMAX_OK;
    if (q == nullptr || o == nullptr) return SOFTMAX_ERR_NULL_POINTER;
    if (nk > 0 && (k == nullptr || v == nullptr)) return SOFTMAX_ERR_NULL_POINTER;  // nk == 0: never read
    const int64_t bh = batch * heads;
    if (heads > 65535 / (batch > 0 ? batch : 1) || bh > 65535) return SOFTMAX_ERR_BAD_SHAPE;
    if (nq > (int64_t(1) << 30) || nq > (int64_t(1) << 40) / head_dim / bh || nk > (int64_t(1) << 40) / head_dim / bh)
        return SOFTMAX_ERR_BAD_SHAPE;
    for (const void* p : {q, k, v, static_cast<const void*>(o)})
        if (uintptr_t(p) % 16) return SOFTMAX_ERR_BAD_SHAPE;
    const uint64_t qbytes = uint64_t(bh * nq * head_dim) * 2, kbytes = uint64_t(bh * nk * head_dim) * 2;
    const uintptr_t ob = uintptr_t(o);
    const struct { uintptr_t p; uint64_t n; } ins[3] = {{uintptr_t(q), qbytes}, {uintptr_t(k), kbytes}, {uintptr_t(v), kbytes}};
    for (const auto& in : ins)
        if (in.n && ob < in.p + in.n && in.p < ob + qbytes) return SOFTMAX_ERR_OVERLAP;

    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.nq = nq;
    a.nk = nk;
    a.offset = nk - nq;
    a.coef = float(double(scale) * kLog2eD);
    const void* fn = dtype == SOFTMAX_F16 ? pick<rws::F16>(head_dim, causal) : pick<rws::BF16>(head_dim, causal);
    const dim3 grid(unsigned((nq + kBM - 1) / kBM), unsigned(bh));
    void* args[] = {&a};
    if (hipLaunchKernel(fn, grid, dim3(kThreads), args, 0, static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipGetLastError();
        return SOFTMAX_ERR_HIP;
    }
    return SOFTMAX_OK;
}
