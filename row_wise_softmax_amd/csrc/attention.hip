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
// each wave owns 16 queries and keeps their Q fragments in registers.  Per
// block of 64 keys the workgroup stages K (row-major) and V (transposed) in
// LDS; each wave computes its 64 x 16 transposed score tile with MFMA,
// updates m and l in fp32 (exponentials as 2^(x log2 e) on v_exp_f32),
// rounds P to the input type in registers and accumulates O^T += V^T P^T.
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
static_assert(kBN * 64 / 8 % kThreads == 0 && (kBN / 2) * (64 / 8) % kThreads == 0, "K/V staging splits evenly");
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

// Exchange with lane ^ 32 (ds_bpermute: byte address of the source lane).
__device__ inline float xor32(float v) {
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, v)));
}

// All-reduce over the four lanes L, L ^ 16, L ^ 32, L ^ 48 (same L % 16).
template <class Op>
__device__ inline float across_groups(float v) {
    v = Op::apply(v, rws::swap16(v));
    return Op::apply(v, xor32(v));
}

__device__ inline unsigned pack2(unsigned short lo, unsigned short hi) { return unsigned(lo) | (unsigned(hi) << 16); }

// Scores are computed transposed, S^T = K Q^T, so that lane L owns query
// c = L % 16 of its wave and holds keys 4g .. 4g + 3 (g = L / 16) of every
// 16-key tile: the softmax statistics of a query are per-lane scalars (shared
// by the four lanes of one query), and the exponentials are already the B
// operand of O^T = V^T P^T -- slot j of a 32-key step takes key 4g + j of its
// first tile (j < 4) or 16 + 4g + (j - 4) of its second, and V^T is read from
// LDS in the same slot order.  While a block is computed, the next block's K
// and V are already on their way from HBM into registers.
template <class E, int D, bool Causal>
__global__ void __launch_bounds__(kThreads) attention_fwd_kernel(AttnArgs a) {
    constexpr int kKS = D / 32;               // MFMA k-steps over the head dimension
    constexpr int kKP = D + 8;                // padded K row in LDS (halves)
    constexpr int kVP = kBN + 8;              // padded V^T row (keys)
    constexpr int kDT = D / 16;               // 16-row output tiles (of O^T) per wave
    constexpr int kLoadsK = kBN * D / 8 / kThreads;        // 16-byte K pieces per thread per block
    constexpr int kLoadsV = (kBN / 2) * (D / 8) / kThreads;  // (key pair, 8 dims) V items per thread
    __shared__ __attribute__((aligned(16))) unsigned short sK[kBN * kKP];
    __shared__ __attribute__((aligned(16))) unsigned short sVt[D * kVP];

    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int w = t / kWave;
    const int g = lane >> 4;
    const int c = lane & 15;
    const int64_t bh = blockIdx.y;
    const int64_t m0 = int64_t(blockIdx.x) * kBM;
    const int64_t qi = m0 + 16 * w + c;  // this lane's query
    const unsigned short* qb = static_cast<const unsigned short*>(a.q) + bh * a.nq * D;
    const unsigned short* kb = static_cast<const unsigned short*>(a.k) + bh * a.nk * D;
    const unsigned short* vb = static_cast<const unsigned short*>(a.v) + bh * a.nk * D;
    unsigned short* ob = static_cast<unsigned short*>(a.o) + bh * a.nq * D;

    // Q fragments (B operand of S^T): column qi, head-dim slots 32s + 8g .. + 7.
    u32x4 qf[kKS];
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
        if (qi < a.nq) qf[s] = rws::ld<true>(reinterpret_cast<const u32x4*>(qb + qi * D + 32 * s + 8 * g));
        else qf[s] = u32x4{0, 0, 0, 0};
    }

    float m = -INFINITY;  // running max of this lane's query (log2 domain)
    float l = 0.0f;       // this lane's partial normaliser (its keys only)
    f32x4 oacc[kDT];
#pragma unroll
    for (int u = 0; u < kDT; ++u) oacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};

    int64_t kend = a.nk;  // keys any query of this workgroup may see
    if (Causal) {
        const int64_t last = m0 + kBM - 1 + a.offset + 1;
        kend = last < kend ? last : kend;
    }

    // K / V staging registers.  K: thread t moves 16-byte pieces t + 256 i
    // (row-major, coalesced).  V: item t + 256 i is a pair of consecutive keys
    // (2 (item % 32), + 1) and 8 head dims (8 (item / 32) ..); the pair is
    // written to V^T as one dword per head dim, so a wave's 32-bit LDS writes
    // cover 32 consecutive dwords of one V^T row per half-wave, the two halves
    // 8 rows (32 banks) apart: no bank conflicts.
    u32x4 kreg[kLoadsK], vreg[kLoadsV][2];
    auto fetch = [&](int64_t n0) {
#pragma unroll
        for (int i = 0; i < kLoadsK; ++i) {
            const int idx = t + i * kThreads;
            const int key = idx / (D / 8);
            const int dc = (idx % (D / 8)) * 8;
            if (n0 + key < a.nk) kreg[i] = rws::ld<false>(reinterpret_cast<const u32x4*>(kb + (n0 + key) * D + dc));
            else kreg[i] = u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < kLoadsV; ++i) {
            const int item = t + i * kThreads;
            const int key = 2 * (item % (kBN / 2));
            const int dc = (item / (kBN / 2)) * 8;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (n0 + key + h < a.nk)
                    vreg[i][h] = rws::ld<false>(reinterpret_cast<const u32x4*>(vb + (n0 + key + h) * D + dc));
                else
                    vreg[i][h] = u32x4{0, 0, 0, 0};
            }
        }
    };
    if (kend > 0) fetch(0);

    for (int64_t n0 = 0; n0 < kend; n0 += kBN) {
        __syncthreads();  // every wave is done reading the previous block from LDS
#pragma unroll
        for (int i = 0; i < kLoadsK; ++i) {
            const int idx = t + i * kThreads;
            const int key = idx / (D / 8);
            const int dc = (idx % (D / 8)) * 8;
            *reinterpret_cast<u32x4*>(sK + key * kKP + dc) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < kLoadsV; ++i) {
            const int item = t + i * kThreads;
            const int key = 2 * (item % (kBN / 2));
            const int dc = (item / (kBN / 2)) * 8;
            unsigned* col = reinterpret_cast<unsigned*>(sVt + dc * kVP + key);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const unsigned a0 = vreg[i][0][e], a1 = vreg[i][1][e];
                col[(2 * e) * (kVP / 2)] = (a0 & 0xffffu) | (a1 << 16);            // head dim dc + 2e
                col[(2 * e + 1) * (kVP / 2)] = (a0 >> 16) | (a1 & 0xffff0000u);    // head dim dc + 2e + 1
            }
        }
        __syncthreads();
        if (n0 + kBN < kend) fetch(n0 + kBN);  // in flight while this block is computed

        // S^T tiles: keys 16nt + 4g + r (r = 0..3) against query qi.
        f32x4 sacc[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
            sacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < kKS; ++s)
                sacc[nt] = mfma<E>(lds16(sK + (16 * nt + c) * kKP + 32 * s + 8 * g), qf[s], sacc[nt]);
        }

        // Scale into the log2 domain; mask only blocks that need it (uniform branch).
        const bool full = n0 + kBN <= a.nk && (!Causal || n0 + kBN - 1 <= m0 + a.offset);
        float bm = -INFINITY;
        if (full) {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sacc[nt][r] *= a.coef;
                    bm = fmaxf(bm, sacc[nt][r]);
                }
        } else {
#pragma unroll
            for (int nt = 0; nt < 4; ++nt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t kj = n0 + 16 * nt + 4 * g + r;
                    float x = sacc[nt][r] * a.coef;
                    if (kj >= a.nk || (Causal && kj > qi + a.offset)) x = -INFINITY;
                    sacc[nt][r] = x;
                    bm = fmaxf(bm, x);
                }
        }
        bm = across_groups<rws::OpMax>(bm);
        const float mnew = fmaxf(m, bm);
        const float msafe = mnew == -INFINITY ? 0.0f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(m - msafe);  // 0 while the query had no key
        m = mnew;
        float ps = 0.0f;
        unsigned short ph[4][4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(sacc[nt][r] - msafe);
                ps += p;
                ph[nt][r] = rws::narrow_half<E>(p);
            }
        l = l * alpha + ps;
#pragma unroll
        for (int u = 0; u < kDT; ++u) oacc[u] *= alpha;

        // O^T += V^T P^T over the block's two 32-key steps.
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const u32x4 pb = {pack2(ph[2 * s][0], ph[2 * s][1]), pack2(ph[2 * s][2], ph[2 * s][3]),
                              pack2(ph[2 * s + 1][0], ph[2 * s + 1][1]), pack2(ph[2 * s + 1][2], ph[2 * s + 1][3])};
#pragma unroll
            for (int u = 0; u < kDT; ++u) {
                const unsigned short* vrow = sVt + (16 * u + c) * kVP + 32 * s + 4 * g;
                const rws::u32x2 lo = *reinterpret_cast<const rws::u32x2*>(vrow);
                const rws::u32x2 hi = *reinterpret_cast<const rws::u32x2*>(vrow + 16);
                const u32x4 va = {lo.x, lo.y, hi.x, hi.y};
                oacc[u] = mfma<E>(va, pb, oacc[u]);
            }
        }
    }

    // Normalise and store: lane holds O[qi][16u + 4g + r], r = 0..3 (8 bytes).
    l = across_groups<rws::OpSum>(l);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (qi < a.nq) {
#pragma unroll
        for (int u = 0; u < kDT; ++u) {
            const rws::u32x2 pk = {pack2(rws::narrow_half<E>(oacc[u][0] * inv), rws::narrow_half<E>(oacc[u][1] * inv)),
                                   pack2(rws::narrow_half<E>(oacc[u][2] * inv), rws::narrow_half<E>(oacc[u][3] * inv))};
            rws::st<true>(reinterpret_cast<rws::u32x2*>(ob + qi * D + 16 * u + 4 * g), pk);
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
