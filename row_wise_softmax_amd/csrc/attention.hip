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
// products run on the matrix cores: v_mfma_f32_32x32x16_{f16,bf16}.
//
// Work split: one workgroup of 4 waves per (batch*head, block of 128
// queries); each wave owns 32 queries and keeps their Q fragments in
// registers.  Per block of 64 keys the workgroup stages K and V (both
// row-major, rows XOR-swizzled) in LDS; each wave computes its 64 x 32
// transposed score tile with MFMA, updates the row statistics in fp32
// (exponentials as 2^(x log2 e) on v_exp_f32), rounds P to the input type in
// registers and accumulates O^T += V^T P^T, reading its V^T operands with
// the transposing LDS load.  The 32 x 32 x 16 product does twice the work of a
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

// 4 waves and 64-key blocks: two workgroups share a CU (80 KB of LDS each).
// 8 waves sharing 128-key blocks (one workgroup of 160 KB per CU, half the
// barriers per key) gives the same results but measured 3-6% slower.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;        // queries per workgroup (32 per wave)
constexpr int kBN = 64;                 // keys per block
constexpr int kTiles = kBN / 32;        // 32-key tiles per block
constexpr int kResident = 8 / kWaves;   // workgroups per CU (two waves per SIMD)
constexpr int kXcds = 8;  // workgroup i runs on XCD i % 8
static_assert(kBN % 32 == 0 && (kBN * 64 * 2 / 1024) % (kThreads / 64) == 0, "K/V blocks split into whole 1 KB pieces per wave");
constexpr double kLog2eD = 1.4426950408889634074;
// The exponent offset m of a query is only moved when a block's max exceeds
// it by more than this (log2 domain), so P <= 2^kSlack: the rescale of the
// accumulators is skipped for most blocks and P stays far inside fp16 range.
constexpr float kSlack = 8.0f;
constexpr int kRsrcWord3 = 0x00020000;  // buffer resource flags word (raw, untyped 32-bit data)
constexpr int kWaitVm0 = 0x0F70;        // s_waitcnt vmcnt(0), other counters untouched

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int64_t nq;
    int64_t nk;
    int64_t offset;  // causal: query i keeps keys j <= i + offset (offset = nk - nq)
    int nqb;         // query blocks per (batch, head)
    int nbh;         // batch * heads
    int grp;         // (batch, head) pairs per scheduling group
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

// v_permlane32_swap (gfx950) swaps lanes 32..63 of its first operand with
// lanes 0..31 of its second (measured on the part).  Given v twice it
// returns, in every lane L, {v[L % 32], v[L % 32 + 32]} in that order: the
// values of lanes L and L ^ 32, with no LDS round trip, whose max and sum come
// out bit-identical in both lanes.  (Each element is copied out before the
// bit cast: a bit cast of the subscripted result read element 0 twice.)
__device__ inline void pair_of(float v, float* lo, float* hi) {
    const int b = __builtin_bit_cast(int, v);
    const auto r = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    const int r0 = r[0], r1 = r[1];
    *lo = __builtin_bit_cast(float, r0);
    *hi = __builtin_bit_cast(float, r1);
}
__device__ inline float pair_max(float v) {
    float lo, hi;
    pair_of(v, &lo, &hi);
    return fmaxf(lo, hi);
}
__device__ inline float pair_sum(float v) {
    float lo, hi;
    pair_of(v, &lo, &hi);
    return lo + hi;
}

// Two fp32 -> one dword of the input type, round to nearest even.
template <class E>
__device__ inline unsigned pack2f(float lo, float hi) {
    const float f[2] = {lo, hi};
    return rws::narrow_dword<E>(f);
}

typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));

// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane j receives,
// as its element e, element j % 4 of the 8 bytes addressed by lane
// 4e + j / 4 of the group.  So if lane s of the group addresses the four
// consecutive head dims 4 (s % 4) .. of key row s / 4, lane j receives head
// dim j of key rows 0, 1, 2, 3: one V^T operand column from row-major V.
__device__ inline rws::u32x2 lds_tr(const unsigned short* p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(rws::u32x2, r);
}

// Scores are computed transposed, S^T = K Q^T, so that lane L owns query
// c = L % 32 of its wave and holds keys 8 (r / 4) + 4 h + r % 4 (h = L / 32,
// r = 0..15) of every 32-key tile: the softmax statistics of a query are
// per-lane scalars (shared by lanes L and L ^ 32), and accumulators 8q .. 8q + 7
// of a tile are already the B operand of the O^T = V^T P^T step over its keys
// 16q .. 16q + 15.  The matching V^T operand is read from row-major V with
// two transposing LDS reads.
//
// The wave works through 32-key tiles in a software pipeline: while the
// vector ALUs turn tile t's scores into P, the matrix cores already compute
// tile t + 1's scores, then P V of tile t runs, then tile t + 1's max is
// taken.  K is therefore needed one 64-key block ahead of V.  K and V go from
// HBM straight into LDS (buffer loads with the lds flag, no registers): K into
// three rotating buffers, V into two, so that the next blocks land while the
// current ones are read, with one barrier per block.  Rows are not padded:
// each row's 16-byte chunks are stored XOR-swizzled so that every LDS read of
// a wave touches distinct banks.
template <class E, int D, bool Causal>
__global__ void __launch_bounds__(kThreads, kResident) attention_fwd_kernel(AttnArgs a) {
    constexpr int kKS = D / 16;                                    // MFMA k-steps over the head dimension
    constexpr int kC = D / 8;                                      // 16-byte chunks per K or V row
    constexpr int kDT = D / 32;                                    // 32-row output tiles (of O^T) per wave
    constexpr int kDma = kBN * D * 2 / 1024 / (kThreads / kWave);  // 1 KB pieces per wave per block
    // Separate arrays, each named statically below: loads from one are then
    // known not to alias the pieces in flight into another, and the compiler
    // does not make them wait for those.
    __shared__ __attribute__((aligned(16))) unsigned short sK0[kBN * D];
    __shared__ __attribute__((aligned(16))) unsigned short sK1[kBN * D];
    __shared__ __attribute__((aligned(16))) unsigned short sK2[kBN * D];
    __shared__ __attribute__((aligned(16))) unsigned short sV0[kBN * D];
    __shared__ __attribute__((aligned(16))) unsigned short sV1[kBN * D];
    // Chunk cc of K row r sits at position cc ^ ksw(r): a K read takes one
    // chunk of 16 consecutive rows.  A V read takes two chunks of 4
    // consecutive rows (and another two per half-wave), so V rows are
    // swizzled by whole 4-chunk groups.  A 128-byte row (D = 64) spans half
    // the banks, so pairs of rows share a pattern.
    auto ksw = [](int r) { return (D == 64 ? r >> 1 : r) & (kC - 1); };
    auto vsw = [](int r) { return D == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3); };

    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(t / kWave);
    const int h = lane >> 5;
    const int c = lane & 31;
    const int swz = ksw(c);  // = ksw(32 half + c) for both tile halves

    // Workgroups of one (batch, head) share K and V: give each XCD (and its
    // L2) a contiguous run j of them, in groups of `grp` (batch, head) pairs,
    // about as many workgroups as an XCD holds at once.  Within a group the
    // causal query blocks run longest-first across all its pairs, so the
    // short ones fill in behind the long ones.
    const int i = blockIdx.x;
    const int full_rounds = a.nwg / kXcds * kXcds;
    const int j = i < full_rounds ? (i % kXcds) * (a.nwg / kXcds) + i / kXcds : i;
    const int gsz = a.grp * a.nqb;  // workgroups per group
    const int g = j / gsz, r = j % gsz;
    const int gb = a.nbh - g * a.grp < a.grp ? a.nbh - g * a.grp : a.grp;  // pairs in this group
    const int64_t bh = int64_t(g) * a.grp + r % gb;
    const int qblk = Causal ? a.nqb - 1 - r / gb : r / gb;
    const int64_t m0 = int64_t(qblk) * kBM;
    const int64_t mw = m0 + 32 * w;  // first query of this wave
    const int64_t qi = mw + c;       // this lane's query
    const unsigned short* qb = static_cast<const unsigned short*>(a.q) + bh * a.nq * D;
    unsigned short* ob = static_cast<unsigned short*>(a.o) + bh * a.nq * D;
    // K and V of this (batch, head) as buffer resources: reads past the last
    // key return zeros (the host guarantees nk * D * 2 < 2^31).
    const uint32_t kvbytes = uint32_t(a.nk * D * 2);
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(static_cast<const unsigned short*>(a.k) + bh * a.nk * D), 0, kvbytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned short*>(static_cast<const unsigned short*>(a.v) + bh * a.nk * D), 0, kvbytes, kRsrcWord3);

    // Q fragments (B operand of S^T): column qi, head-dim slots 16s + 8h .. + 7.
    u32x4 qf[kKS];
#pragma unroll
    for (int s = 0; s < kKS; ++s) {
        if (qi < a.nq) qf[s] = rws::ld<false>(reinterpret_cast<const u32x4*>(qb + qi * D + 16 * s + 8 * h));
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
    int64_t kend = a.nk, wend = mw < a.nq ? a.nk : 0;  // a wave wholly past the last query sees nothing
    if (Causal) {
        kend = qlast + a.offset + 1 < kend ? qlast + a.offset + 1 : kend;
        wend = mw + 31 + a.offset + 1 < wend ? mw + 31 + a.offset + 1 : wend;
        wend = wend < kend ? wend : kend;  // never past the staged blocks
    }
    const int64_t nblk = kend > 0 ? (kend + kBN - 1) / kBN : 0;
    // Keys this lane's query keeps: j < kmax.
    const int64_t kmax = Causal && qi + a.offset + 1 < a.nk ? qi + a.offset + 1 : a.nk;

    // One 64-key block of K or V into LDS: each wave moves kDma 1 KB pieces;
    // lane L of a piece fills position L % kC of row (piece rows) + L / kC, so
    // it fetches the chunk that the swizzle puts there.  Rows past the last
    // key read as zeros.
    auto dma = [&](__amdgpu_buffer_rsrc_t rs, int64_t n0, unsigned short* dst, auto sw) {
#pragma unroll
        for (int i = 0; i < kDma; ++i) {
            const int piece = w * kDma + i;  // wave-uniform
            const int row = piece * (512 / D) + lane / kC;
            const int chunk = (lane % kC) ^ sw(row);
            const uint32_t off = uint32_t(((n0 + row) * D + chunk * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + piece * 512),
                                                     16, off, 0, 0, 0);
        }
    };
    // V rows past the last key must hold zeros, not stale LDS (P is 0 there,
    // and 0 * NaN would not be): clear them in the one block that has such
    // rows, before its pieces are requested (those rows then read as zeros too).
    auto clear_v_tail = [&](int64_t n0, unsigned short* dst) {
        const int64_t valid = a.nk - n0;
        if (valid >= kBN) return;
        for (int idx = t; idx < kBN * kC; idx += kThreads)
            if (idx / kC >= valid) *reinterpret_cast<u32x4*>(dst + idx * 8) = u32x4{0, 0, 0, 0};
    };

    // S^T of one 32-key tile (keys 32 half + 8(r/4) + 4h + r%4 of a staged block).
    // The lane's K read offset of every k-step, computed once.
    int koff[kKS];
#pragma unroll
    for (int s = 0; s < kKS; ++s) koff[s] = c * D + ((2 * s + h) ^ swz) * 8;
    auto scores = [&](const unsigned short* blk, int half) {
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
        for (int s = 0; s < kKS; ++s) acc = mfma<E>(lds16(blk + 32 * half * D + koff[s]), qf[s], acc);
        return acc;
    };
    // Mask a tile starting at key k0, then move the exponent offset if its max
    // would make P exceed 2^kSlack (the accumulators are rescaled to match).
    auto prepare = [&](f32x16& sc, int64_t k0) {
        const bool full = k0 + 32 <= a.nk && (!Causal || k0 + 31 <= mw + a.offset);  // wave-uniform
        if (!full) {
            // A real branch (the barrier keeps the compiler from flattening it
            // into selects that every tile would pay for).  Accumulator r
            // holds key k0 + 4h + 8(r/4) + r%4, kept iff that is < kmax.
            __builtin_amdgcn_sched_barrier(0);
            const int64_t room = kmax - k0 - 4 * h;
            const int lim = room < 0 ? 0 : room > 32 ? 32 : int(room);
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r >> 2) + (r & 3) >= lim) sc[r] = -INFINITY;
        }
        float bm = sc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) bm = fmaxf(bm, sc[r]);
        bm = pair_max(bm) * a.coef;  // the query's tile max, log2 domain
        if (__builtin_amdgcn_ballot_w64(bm > m + kSlack)) {
            const float mnew = fmaxf(m, bm);
            const float alpha = mnew == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m - mnew);  // m = -inf: 0
            m = mnew;
            l *= alpha;
#pragma unroll
            for (int u = 0; u < kDT; ++u) oacc[u] *= alpha;
        }
    };
    // V^T operand for output tile u and the 8 key slots of this lane in a
    // 16-key step starting at key kb of the block: slots e < 4 are keys
    // kb + 4h + e, slots e >= 4 keys kb + 8 + 4h + (e - 4).  Lane s of each
    // 16-lane group addresses key row (s / 4) of those four and head dims
    // 32u + 16 (group % 2) + 4 (s % 4) .. + 3.
    const int grp = lane >> 4, sl = lane & 15;
    auto v_operand = [&](const unsigned short* blk, int kb, int u) {
        const int dim = 32 * u + 16 * (grp & 1) + 4 * (sl & 3);
        const int r0 = kb + 4 * h + (sl >> 2), r1 = r0 + 8;
        const rws::u32x2 lo = lds_tr(blk + r0 * D + (((dim >> 3) ^ vsw(r0)) << 3) + (dim & 7));
        const rws::u32x2 hi = lds_tr(blk + r1 * D + (((dim >> 3) ^ vsw(r1)) << 3) + (dim & 7));
        return u32x4{lo.x, lo.y, hi.x, hi.y};
    };
    // P = 2^(s coef - m) rounded to the input type; O^T += V^T P^T over the
    // tile's two 16-key steps.
    auto consume = [&](const f32x16& sc, const unsigned short* vblk, int half) {
        const float moff = m == -INFINITY ? 0.0f : m;  // no visible key yet: every score is -inf
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[r], a.coef, -moff));
            l += p[r];
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const u32x4 pb = {pack2f<E>(p[8 * q], p[8 * q + 1]), pack2f<E>(p[8 * q + 2], p[8 * q + 3]),
                              pack2f<E>(p[8 * q + 4], p[8 * q + 5]), pack2f<E>(p[8 * q + 6], p[8 * q + 7])};
#pragma unroll
            for (int u = 0; u < kDT; ++u) oacc[u] = mfma<E>(v_operand(vblk, 32 * half + 16 * q, u), pb, oacc[u]);
        }
    };

    f32x16 scur;
    if (nblk > 0) {
        clear_v_tail(0, sV0);
        dma(krs, 0, sK0, ksw);
        if (nblk > 1) dma(krs, kBN, sK1, ksw);
        dma(vrs, 0, sV0, vsw);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this wave's pieces have landed
        __syncthreads();
        if (wend > 0) {
            scur = scores(sK0, 0);
            prepare(scur, 0);
        }
    }
    // Block jb: K block jb in kcur, jb + 1 in knext, jb + 2 goes to kfar; V
    // block jb in vcur, jb + 1 goes to vnext.
    auto block = [&](int64_t jb, const unsigned short* kcur, const unsigned short* knext, unsigned short* kfar,
                     const unsigned short* vcur, unsigned short* vnext) {
        const int64_t n0 = jb * kBN;
        if (jb > 0) {
            __builtin_amdgcn_s_waitcnt(kWaitVm0);  // K block jb + 1 and V block jb have landed
            __syncthreads();  // ... for every wave; all are done with K block jb - 1 and V block jb - 1
        }
        if (jb + 2 < nblk) dma(krs, n0 + 2 * kBN, kfar, ksw);  // in flight while this block is computed
        if (jb + 1 < nblk) {
            clear_v_tail(n0 + kBN, vnext);
            dma(vrs, n0 + kBN, vnext, vsw);
        }
#pragma unroll
        for (int half = 0; half < kTiles; ++half) {
            const int64_t k0 = n0 + 32 * half;  // this tile's first key
            if (k0 < wend) {                    // wave-uniform: some key of the tile is visible
                // Next tile's scores (always from staged LDS; discarded past the last tile).
                f32x16 snext = half + 1 < kTiles ? scores(kcur, half + 1) : scores(knext, 0);
                consume(scur, vcur, half);
                if (k0 + 32 < wend) prepare(snext, k0 + 32);
                scur = snext;  // unused when the next tile is past wend
            }
        }
    };
    // Six-block cycle: the K buffer index cycles with period 3, the V one with 2.
    for (int64_t jb = 0; jb < nblk; jb += 6) {
        block(jb, sK0, sK1, sK2, sV0, sV1);
        if (jb + 1 < nblk) block(jb + 1, sK1, sK2, sK0, sV1, sV0);
        if (jb + 2 < nblk) block(jb + 2, sK2, sK0, sK1, sV0, sV1);
        if (jb + 3 < nblk) block(jb + 3, sK0, sK1, sK2, sV1, sV0);
        if (jb + 4 < nblk) block(jb + 4, sK1, sK2, sK0, sV0, sV1);
        if (jb + 5 < nblk) block(jb + 5, sK2, sK0, sK1, sV1, sV0);
    }

    // Normalise and store: lane holds O[qi][32u + 8j + 4h + r], r = 0..3 (8 bytes).
    l = pair_sum(l);
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (qi < a.nq) {
#pragma unroll
        for (int u = 0; u < kDT; ++u)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const rws::u32x2 pk = {pack2f<E>(oacc[u][4 * jj] * inv, oacc[u][4 * jj + 1] * inv),
                                       pack2f<E>(oacc[u][4 * jj + 2] * inv, oacc[u][4 * jj + 3] * inv)};
                rws::st<false>(reinterpret_cast<rws::u32x2*>(ob + qi * D + 32 * u + 8 * jj + 4 * h), pk);
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
    if (nk * head_dim * 2 >= (int64_t(1) << 31)) return SOFTMAX_ERR_BAD_SHAPE;  // K/V of one head < 2 GiB
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
    a.nbh = int(bh);
    // Group about one XCD's worth of resident workgroups (32 CUs x kResident).
    const int64_t per_group = 32 * kResident / nqb > 1 ? 32 * kResident / nqb : 1;
    a.grp = int(per_group < bh ? per_group : bh);
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
