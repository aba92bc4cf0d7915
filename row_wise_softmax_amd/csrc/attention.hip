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
// Work split: one workgroup of 4 waves per (batch*head, block of 128
// queries); each wave owns 32 queries and keeps their Q fragments in
// registers.  Per block of 64 keys the workgroup stages K (row-major) and V
// (transposed) in LDS; each wave computes its 64 x 32 transposed score tile
// with MFMA, updates the row statistics in fp32 (exponentials as 2^(x log2 e)
// on v_exp_f32), rounds P to the input type in registers and accumulates
// O^T += V^T P^T.  The 32 x 32 x 16 product does twice the work of a
// 16 x 16 x 32 one for the same 16 bytes of operand per lane, so every K or V
// fragment read from LDS feeds twice as many flops: LDS bandwidth, not the
// matrix cores, is what bounds a wave that owns only 16 queries.
//
// MFMA operand layout used (32 x 32 x 16): lane L supplies row (or column)
// L % 32 and eight consecutive k slots 8 (L / 32) .. 8 (L / 32) + 7; the
// 32 x 32 fp32 result lands with column L % 32 and, in accumulator r
// (0..15), row 8 (r / 4) + 4 (L / 32) + r % 4.  Both operands of every
// product are filled with the same slot -> k assignment, so the sum over k is
// the same whatever order the hardware walks the slots in.
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
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;  // queries per workgroup (32 per wave)
constexpr int kBN = 64;   // keys per block
constexpr int kThreads = 256;
constexpr int kXcds = 8;  // workgroup i runs on XCD i % 8
static_assert(kBN * 64 / 8 % kThreads == 0 && (kBN / 2) * (64 / 8) % kThreads == 0, "K/V staging splits evenly");
constexpr double kLog2eD = 1.4426950408889634074;
// The exponent offset m of a query is only moved when a block's max exceeds
// it by more than this (log2 domain), so P <= 2^kSlack: the rescale of the
// accumulators is skipped for most blocks and P stays far inside fp16 range.
constexpr float kSlack = 8.0f;

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int64_t nq;
    int64_t nk;
    int64_t offset;  // causal: query i keeps keys j <= i + offset (offset = nk - nq)
    int nqb;         // query blocks per (batch, head)
    int nwg;         // workgroups in the grid
    float coef;      // scale * log2(e)
};

template <class E>
__device__ inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    if constexpr (std::is_same_v<E, rws::F16>)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ inline u32x4 lds16(const unsigned short* p) { return *reinterpret_cast<const u32x4*>(p); }

// Exchange with lane ^ 32 (ds_bpermute: byte address of the source lane).
__device__ inline float xor32(float v) {
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, v)));
}

// Two fp32 -> one dword of the input type, round to nearest even.
template <class E>
__device__ inline unsigned pack2f(float lo, float hi) {
    const float f[2] = {lo, hi};
    return rws::narrow_dword<E>(f);
}

// V^T keeps the 16 keys of each group in the order 0-3, 8-11, 4-7, 12-15
// (bits 2 and 3 of the key swapped), so that the eight keys one lane feeds to
// a 16-key MFMA step are 16 contiguous bytes.  Key pairs stay adjacent:
// this maps the pair index p = key / 2 (bits 1 and 2 swapped).
__device__ inline int vt_pair(int p) { return (p & ~6) | ((p & 2) << 1) | ((p & 4) >> 1); }

// Scores are computed transposed, S^T = K Q^T, so that lane L owns query
// c = L % 32 of its wave and holds keys 8 (r / 4) + 4 h + r % 4 (h = L / 32,
// r = 0..15) of every 32-key tile: the softmax statistics of a query are
// per-lane scalars (shared by lanes L and L ^ 32), and accumulators 8q .. 8q + 7
// of a tile are already the B operand of the O^T = V^T P^T step over its keys
// 16q .. 16q + 15.  While a block is computed, the next block's K and V are
// already on their way from HBM into registers.
template <class E, int D, bool Causal>
__global__ void __launch_bounds__(kThreads, 2) attention_fwd_kernel(AttnArgs a) {
    constexpr int kKS = D / 16;                              // MFMA k-steps over the head dimension
    constexpr int kKP = D + 8;                               // padded K row in LDS (halves)
    constexpr int kVP = kBN + 8;                             // padded V^T row (keys)
    constexpr int kDT = D / 32;                              // 32-row output tiles (of O^T) per wave
    constexpr int kLoadsK = kBN * D / 8 / kThreads;          // 16-byte K pieces per thread per block
    constexpr int kLoadsV = (kBN / 2) * (D / 8) / kThreads;  // (key pair, 8 dims) V items per thread
    __shared__ __attribute__((aligned(16))) unsigned short sK[kBN * kKP];
    __shared__ __attribute__((aligned(16))) unsigned short sVt[D * kVP];

    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int w = t / kWave;
    const int h = lane >> 5;
    const int c = lane & 31;

    // Workgroups of one (batch, head) share K and V: give each XCD (and its
    // L2) a contiguous run of them.  Causal query blocks run longest-first.
    const int i = blockIdx.x;
    const int full_rounds = a.nwg / kXcds * kXcds;
    const int j = i < full_rounds ? (i % kXcds) * (a.nwg / kXcds) + i / kXcds : i;
    const int64_t bh = j / a.nqb;
    const int qblk = Causal ? a.nqb - 1 - j % a.nqb : j % a.nqb;
    const int64_t m0 = int64_t(qblk) * kBM;
    const int64_t mw = m0 + 32 * w;  // first query of this wave
    const int64_t qi = mw + c;       // this lane's query
    const unsigned short* qb = static_cast<const unsigned short*>(a.q) + bh * a.nq * D;
    const unsigned short* kb = static_cast<const unsigned short*>(a.k) + bh * a.nk * D;
    const unsigned short* vb = static_cast<const unsigned short*>(a.v) + bh * a.nk * D;
    unsigned short* ob = static_cast<unsigned short*>(a.o) + bh * a.nq * D;

    // Q fragments (B operand of S^T): column qi, head-dim slots 16s + 8h .. + 7.
    u32x4 qf[kKS];
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
        if (qi < a.nq) qf[s] = rws::ld<true>(reinterpret_cast<const u32x4*>(qb + qi * D + 16 * s + 8 * h));
        else qf[s] = u32x4{0, 0, 0, 0};
    }

    float m = -INFINITY;  // exponent offset of this lane's query (log2 domain)
    float l = 0.0f;       // this lane's partial normaliser (its keys only)
    f32x16 oacc[kDT];
#pragma unroll
    for (int u = 0; u < kDT; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[u][r] = 0.0f;

    // Keys any query of this workgroup (of this wave) may see.
    const int64_t qlast = (m0 + kBM < a.nq ? m0 + kBM : a.nq) - 1;
    int64_t kend = a.nk, wend = a.nk;
    if (Causal) {
        kend = qlast + a.offset + 1 < kend ? qlast + a.offset + 1 : kend;
        wend = mw + 31 + a.offset + 1 < wend ? mw + 31 + a.offset + 1 : wend;
    }
    const bool wave_idle = mw >= a.nq;  // every query of this wave is past the end

    // K / V staging registers.  K: thread t moves 16-byte pieces t + 256 i
    // (row-major, coalesced).  V: item t + 256 i is a pair of consecutive keys
    // (2 (item % 32), + 1) and 8 head dims (8 (item / 32) ..); the pair is
    // written to V^T as one dword per head dim, so a wave's 32-bit LDS writes
    // cover 32 distinct dwords of one V^T row per half-wave, the two halves
    // 8 rows (32 banks) apart.
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
            for (int e = 0; e < 2; ++e) {
                if (n0 + key + e < a.nk)
                    vreg[i][e] = rws::ld<false>(reinterpret_cast<const u32x4*>(vb + (n0 + key + e) * D + dc));
                else
                    vreg[i][e] = u32x4{0, 0, 0, 0};
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
            const int pair = item % (kBN / 2);
            const int dc = (item / (kBN / 2)) * 8;
            unsigned* col = reinterpret_cast<unsigned*>(sVt + dc * kVP) + (pair & ~7) + vt_pair(pair & 7);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const unsigned a0 = vreg[i][0][e], a1 = vreg[i][1][e];
                col[(2 * e) * (kVP / 2)] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);      // head dim dc + 2e
                col[(2 * e + 1) * (kVP / 2)] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);  // head dim dc + 2e + 1
            }
        }
        __syncthreads();
        if (n0 + kBN < kend) fetch(n0 + kBN);  // in flight while this block is computed
        if (wave_idle || n0 >= wend) continue;  // nothing of this block is visible to this wave

        // S^T tiles: keys n0 + 32nt + 8(r/4) + 4h + r%4 against query qi.
        f32x16 sacc[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[nt][r] = 0.0f;
#pragma unroll
            for (int s = 0; s < kKS; ++s)
                sacc[nt] = mfma<E>(lds16(sK + (32 * nt + c) * kKP + 16 * s + 8 * h), qf[s], sacc[nt]);
        }

        // Mask only blocks that need it (wave-uniform branch); block max in raw score units.
        const bool full = n0 + kBN <= a.nk && (!Causal || n0 + kBN - 1 <= mw + a.offset);
        float bm = -INFINITY;
        if (!full) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int64_t kj = n0 + 32 * nt + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (kj >= a.nk || (Causal && kj > qi + a.offset)) sacc[nt][r] = -INFINITY;
                }
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int r = 0; r < 16; ++r) bm = fmaxf(bm, sacc[nt][r]);
        bm = fmaxf(bm, xor32(bm)) * a.coef;  // the query's block max, log2 domain

        // Move the exponent offset only when P would exceed 2^kSlack.
        if (__builtin_amdgcn_ballot_w64(bm > m + kSlack)) {
            const float mnew = fmaxf(m, bm);
            const float alpha = mnew == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - mnew);  // m = -inf: 0
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int u = 0; u < kDT; ++u) oacc[u] *= alpha;
        }
        const float moff = m == -INFINITY ? 0.0f : m;  // no visible key yet: every score is -inf

        // P = 2^(s coef - m), rounded to the input type; O^T += V^T P^T per 16 keys.
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[nt][r], a.coef, -moff));
                l += p[r];
            }
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const u32x4 pb = {pack2f<E>(p[8 * q], p[8 * q + 1]), pack2f<E>(p[8 * q + 2], p[8 * q + 3]),
                                  pack2f<E>(p[8 * q + 4], p[8 * q + 5]), pack2f<E>(p[8 * q + 6], p[8 * q + 7])};
#pragma unroll
                for (int u = 0; u < kDT; ++u)
                    oacc[u] = mfma<E>(lds16(sVt + (32 * u + c) * kVP + 32 * nt + 16 * q + 8 * h), pb, oacc[u]);
            }
        }
    }

    // Normalise and store: lane holds O[qi][32u + 8j + 4h + r], r = 0..3 (8 bytes).
    l += xor32(l);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (qi < a.nq) {
#pragma unroll
        for (int u = 0; u < kDT; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const rws::u32x2 pk = {pack2f<E>(oacc[u][4 * jj] * inv, oacc[u][4 * jj + 1] * inv),
                                       pack2f<E>(oacc[u][4 * jj + 2] * inv, oacc[u][4 * jj + 3] * inv)};
                rws::st<true>(reinterpret_cast<rws::u32x2*>(ob + qi * D + 32 * u + 8 * jj + 4 * h), pk);
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
    const int64_t nqb = (nq + kBM - 1) / kBM;
    if (nqb > INT32_MAX / bh) return SOFTMAX_ERR_BAD_SHAPE;  // one workgroup per (batch*head, 128 queries)
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
    a.nqb = int(nqb);
    a.nwg = int(nqb * bh);
    a.coef = float(double(scale) * kLog2eD);
    const void* fn = dtype == SOFTMAX_F16 ? pick<rws::F16>(head_dim, causal) : pick<rws::BF16>(head_dim, causal);
    void* args[] = {&a};
    if (hipLaunchKernel(fn, dim3(unsigned(a.nwg)), dim3(kThreads), args, 0, static_cast<hipStream_t>(stream)) !=
        hipSuccess) {
        (void)hipGetLastError();
        return SOFTMAX_ERR_HIP;
    }
    return SOFTMAX_OK;
}
