// softmax_kernels.hpp -- HIP kernels (gfx950 / CDNA4) for the fused, numerically
// stable row softmax  y[i,j] = exp(x[i,j] - m_i) / sum_k exp(x[i,k] - m_i),
// m_i = max_k x[i,k], with fp32 accumulation for fp32, fp16 and bf16 data.
//
// The method: fuse max, exp, sum and normalise into one kernel so that each
// element crosses HBM once in and once out ("I Wrote My First GPU Kernel",
// section "What Fusion Actually Does"; "fused-softmax-roofline", the
// row-softmax fragment), subtract the row max first, let masked columns carry
// -inf so they contribute exactly 0 ("GPU Kernels - Implementing and
// optimizing Softmax", section "Baseline & Triton Softmax kernel"), take one
// reciprocal of the sum per row instead of dividing per element (same page,
// section "CUDA optimized for block per row"), and for rows too wide to keep on
// chip use the running-max/rescaled-sum form and its pairwise merge
// ("Dissecting Memory Bandwidth & SRAM Tiling in Triton", section "The
// Mathematical Remedy: Online Softmax Tiling").
//
// Four single-launch kernel shapes, all built on 16-byte coalesced accesses
// and wave64 cross-lane reductions (DPP, ds_swizzle, readlane), with no MFMA
// (there is no contraction here):
//   * packed  -- L lanes of one wave per row (L = 1..64), 64/L rows per wave,
//                G row groups per wave in flight; no LDS, no barrier;
//   * row     -- one workgroup of W waves per row, the row held in registers,
//                one LDS slot per wave for the cross-wave combine;
//   * row_pf  -- the row kernel made persistent: each workgroup loops over
//                rows and prefetches the next row while finishing the current;
//   * online  -- one workgroup per row of any width: pass 1 streams the row in
//                chunks keeping a per-lane (max, sum) pair, pass 2 re-reads,
//                normalises and writes.
// plus the split-row pair (several workgroups per row: per-tile (max, sum)
// into a workspace, then merge and normalise) and a plain copy kernel that
// serves as the bandwidth reference.
//
// Arithmetic (all fp32).  In the single-pass kernels the exponentials are
// 2^(x*c - a) with one FMA and v_exp_f32, where c = scale * log2(e) (scale 1
// for the plain softmax) and a = m * c rounded to fp32 is the row's "frame".
// Every exponential of a row uses the same frame, so the rounding of a
// cancels in the ratio; only the FMA's own rounding of each argument remains.
// Rows with a very large max are first rebased (rebase_large_max) so that
// the rounding of a stays below 1/4.  A row whose entries are all -inf gets
// frame 0, so every exponential is exp2(-inf) = +0, the sum is 0, the
// reciprocal is taken as 0 and every output is +0.  The reciprocal of the sum
// is v_rcp_f32 (about 1 ulp; the sum is at least 1 whenever the row has a
// finite max, since the max itself contributes 1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rws {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 b16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------ element types

struct F32 { static constexpr int kBytes = 4; };
struct F16 { static constexpr int kBytes = 2; };
struct BF16 { static constexpr int kBytes = 2; };

// One memory access of N elements (N * kBytes in {2, 4, 8, 16} bytes).
template <int Bytes> struct RawOf;
template <> struct RawOf<16> { typedef u32x4 type; };
template <> struct RawOf<8> { typedef u32x2 type; };
template <> struct RawOf<4> { typedef unsigned type; };
template <> struct RawOf<2> { typedef unsigned short type; };

template <class E, int N>
struct Access {
    static constexpr int kN = N;
    typedef typename RawOf<N * E::kBytes>::type raw;
};

// Widen one dword holding one fp32 or two 16-bit values.
__device__ inline float u32_as_f32(unsigned d) { return __builtin_bit_cast(float, d); }

template <class E> __device__ inline void widen_dword(unsigned d, float* f);
template <> __device__ inline void widen_dword<F32>(unsigned d, float* f) { f[0] = u32_as_f32(d); }
template <> __device__ inline void widen_dword<F16>(unsigned d, float* f) {
    f[0] = (float)__builtin_bit_cast(_Float16, (unsigned short)(d & 0xffffu));
    f[1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(d >> 16));
}
template <> __device__ inline void widen_dword<BF16>(unsigned d, float* f) {
    f[0] = u32_as_f32(d << 16);           // bf16 is the upper half of an fp32
    f[1] = u32_as_f32(d & 0xffff0000u);
}

// Narrow fp32 -> one dword, rounding to nearest even (v_cvt_pk_*_f32 on gfx950).
template <class E> __device__ inline unsigned narrow_dword(const float* f);
template <> __device__ inline unsigned narrow_dword<F32>(const float* f) { return __builtin_bit_cast(unsigned, f[0]); }
template <> __device__ inline unsigned narrow_dword<F16>(const float* f) {
    f32x2 v = {f[0], f[1]};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, h16x2));
}
template <> __device__ inline unsigned narrow_dword<BF16>(const float* f) {
    f32x2 v = {f[0], f[1]};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, b16x2));
}

template <class E> __device__ inline float widen_half(unsigned short h);
template <> __device__ inline float widen_half<F16>(unsigned short h) { return (float)__builtin_bit_cast(_Float16, h); }
template <> __device__ inline float widen_half<BF16>(unsigned short h) { return u32_as_f32((unsigned)h << 16); }
template <class E> __device__ inline unsigned short narrow_half(float f);
template <> __device__ inline unsigned short narrow_half<F16>(float f) { return __builtin_bit_cast(unsigned short, (_Float16)f); }
template <> __device__ inline unsigned short narrow_half<BF16>(float f) { return __builtin_bit_cast(unsigned short, (__bf16)f); }

// Load / store N elements at p (an address aligned to the access size).
//
// Streaming accesses carry the non-temporal hint (`nt`): every element is read
// once and written once, so neither side should displace other data from L2
// and the Infinity Cache.  On MI355X this raises a plain 16-byte copy of 64 MiB
// from about 5.5 to about 6.0 TB/s.  The online kernel's first pass reads
// with the default policy (Keep = true) so that its second pass can hit.
template <bool NT, class T>
__device__ inline T ld(const T* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    else return *p;
}
template <bool NT, class T>
__device__ inline void st(T* p, T v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

template <class E, int N, bool Keep = false>
__device__ inline void load_elems(const typename Access<E, N>::raw* p, float* f) {
    constexpr int kBytes = N * E::kBytes;
    constexpr bool kNT = !Keep;
    if constexpr (kBytes == 16) {
        u32x4 r = ld<kNT>(p);
        constexpr int per = 4 / E::kBytes;
        widen_dword<E>(r.x, f); widen_dword<E>(r.y, f + per);
        widen_dword<E>(r.z, f + 2 * per); widen_dword<E>(r.w, f + 3 * per);
    } else if constexpr (kBytes == 8) {
        u32x2 r = ld<kNT>(p);
        constexpr int per = 4 / E::kBytes;
        widen_dword<E>(r.x, f); widen_dword<E>(r.y, f + per);
    } else if constexpr (kBytes == 4) {
        widen_dword<E>(ld<kNT>(p), f);
    } else {
        f[0] = widen_half<E>(ld<kNT>(p));
    }
}

template <class E, int N>
__device__ inline void store_elems(typename Access<E, N>::raw* p, const float* f) {
    constexpr int kBytes = N * E::kBytes;
    if constexpr (kBytes == 16) {
        constexpr int per = 4 / E::kBytes;
        u32x4 r = {narrow_dword<E>(f), narrow_dword<E>(f + per), narrow_dword<E>(f + 2 * per),
                   narrow_dword<E>(f + 3 * per)};
        st<true>(p, r);
    } else if constexpr (kBytes == 8) {
        constexpr int per = 4 / E::kBytes;
        u32x2 r = {narrow_dword<E>(f), narrow_dword<E>(f + per)};
        st<true>(p, r);
    } else if constexpr (kBytes == 4) {
        st<true>(p, narrow_dword<E>(f));
    } else {
        st<true>(p, narrow_half<E>(f[0]));
    }
}

// Store one element at p (one of an access's N, element-aligned).
template <class E>
__device__ inline void store_elem(void* p, float f) {
    if constexpr (E::kBytes == 4) st<true>(static_cast<unsigned*>(p), __builtin_bit_cast(unsigned, f));
    else st<true>(static_cast<unsigned short*>(p), narrow_half<E>(f));
}

// ------------------------------------------------------- cross-lane steps

__device__ inline float as_f(int v) { return __builtin_bit_cast(float, v); }
__device__ inline int as_i(float v) { return __builtin_bit_cast(int, v); }

// DPP controls (GFX9 encoding): quad_perm [1,0,3,2] and [2,3,0,1] swap
// neighbours at distance 1 and 2; row_half_mirror reverses each 8-lane half
// row, row_mirror each 16-lane row.  Once every group of 2^k lanes holds one
// value, a mirror pairs each lane with a lane of the sibling group, which is
// all an all-reduce needs.
template <int Ctrl>
__device__ inline float dpp(float v) {
    return as_f(__builtin_amdgcn_update_dpp(0, as_i(v), Ctrl, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// ds_swizzle in bit mode with and_mask 0x1f, xor_mask 0x10: partner = lane ^ 16.
__device__ inline float swap16(float v) { return as_f(__builtin_amdgcn_ds_swizzle(as_i(v), 0x401F)); }

struct OpMax { __device__ static float apply(float a, float b) { return fmaxf(a, b); } };
struct OpSum { __device__ static float apply(float a, float b) { return a + b; } };

// All-reduce over each aligned group of L consecutive lanes (L a power of two
// <= 64).  Every lane of a group ends with the same bits: each step combines a
// lane with a partner holding the same partial, and both operations commute.
template <int L, class Op>
__device__ inline float group_reduce(float v) {
    if constexpr (L >= 2) v = Op::apply(v, dpp<kDppXor1>(v));
    if constexpr (L >= 4) v = Op::apply(v, dpp<kDppXor2>(v));
    if constexpr (L >= 8) v = Op::apply(v, dpp<kDppHalfMirror>(v));
    if constexpr (L >= 16) v = Op::apply(v, dpp<kDppMirror>(v));
    if constexpr (L >= 32) v = Op::apply(v, swap16(v));
    if constexpr (L >= 64) {
        float lo = as_f(__builtin_amdgcn_readlane(as_i(v), 0));
        float hi = as_f(__builtin_amdgcn_readlane(as_i(v), 32));
        v = Op::apply(lo, hi);
    }
    return v;
}

// Merge of two (max, sum) pairs, each sum taken relative to its own max:
//   m = max(m1, m2),  s = s1 * e^(c (m1 - m)) + s2 * e^(c (m2 - m)),
// with c = scale * log2 e applied through exp2; a max of -inf marks an empty
// pair (sum 0).
__device__ inline float exp_diff(float d, float coef) { return __builtin_amdgcn_exp2f(d * coef); }

__device__ inline void merge_pair(float& m, float& s, float m2, float s2, float coef) {
    float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;  // both empty
    s = s * exp_diff(m - mn, coef) + s2 * exp_diff(m2 - mn, coef);
    m = mn;
}

template <int Ctrl>
__device__ inline void pair_step_dpp(float& m, float& s, float coef) {
    merge_pair(m, s, dpp<Ctrl>(m), dpp<Ctrl>(s), coef);
}

// All-reduce of (max, sum) pairs over a whole wave.
__device__ inline void wave_reduce_pair(float& m, float& s, float coef) {
    pair_step_dpp<kDppXor1>(m, s, coef);
    pair_step_dpp<kDppXor2>(m, s, coef);
    pair_step_dpp<kDppHalfMirror>(m, s, coef);
    pair_step_dpp<kDppMirror>(m, s, coef);
    merge_pair(m, s, swap16(m), swap16(s), coef);
    float m_lo = as_f(__builtin_amdgcn_readlane(as_i(m), 0));
    float s_lo = as_f(__builtin_amdgcn_readlane(as_i(s), 0));
    float m_hi = as_f(__builtin_amdgcn_readlane(as_i(m), 32));
    float s_hi = as_f(__builtin_amdgcn_readlane(as_i(s), 32));
    merge_pair(m_lo, s_lo, m_hi, s_hi, coef);
    m = m_lo;
    s = s_lo;
}

// The row's frame from its max: m * c (c = scale * log2 e), or 0 for an all
// -inf row.
__device__ inline float frame_of(float m, float coef) { return m == -INFINITY ? 0.0f : m * coef; }

// exp2(fma(x, c, -frame)) with frame = fl(m c): for x = m the argument is the
// rounding error of fl(m c), at most ulp(m c) / 2.  It is common to the whole
// row and cancels in the ratio, but it must stay small: a large one both
// overflows exp2 and inflates every other argument's own rounding.  Up to
// |m c| = 2^22 it is at most 0.25.
constexpr float kFrameLimit = 4194304.0f;  // 2^22
__device__ inline bool frame_small(float m, float coef) {
    return m == -INFINITY || fabsf(m * coef) <= kFrameLimit;
}

__device__ inline float exp_in_frame(float x, float coef, float frame) {
    return __builtin_amdgcn_exp2f(__builtin_fmaf(x, coef, -frame));
}

// Rows whose max has |m c| > 2^22 (for scale 1, |m| above about 2.9e6) are
// rebased in registers, x := x - m and m := 0, before the one-FMA path.  The
// subtraction is exact for every x within a factor of two of m (the entries
// whose exponentials matter), x = m becomes exactly 0, and x - m may overflow
// to -inf only where e^(c (x - m)) is 0 anyway.  The test is a ballot, so
// ordinary rows pay one scalar branch.
template <int n>
__device__ inline void rebase_large_max(float* x, float& m, float coef) {
    if (__builtin_amdgcn_ballot_w64(!frame_small(m, coef)) != 0) {
        if (!frame_small(m, coef)) {
#pragma unroll
            for (int i = 0; i < n; ++i) x[i] = x[i] - m;
            m = 0.0f;
        }
    }
}

// Replace x[0..n) by its exponentials relative to the row max m; returns
// their sum.  Requires frame_small(m, coef) (see rebase_large_max).
template <int n>
__device__ inline float exp_and_sum(float* x, float m, float coef) {
    const float fr = frame_of(m, coef);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < n; ++i) {
        x[i] = exp_in_frame(x[i], coef, fr);
        s += x[i];
    }
    return s;
}

// 1 / s for s >= 1 (a row with a finite max always has s >= 1), 0 for s == 0.
__device__ inline float recip_sum(float s) { return s > 0.0f ? __builtin_amdgcn_rcpf(s) : 0.0f; }

// ---------------------------------------------------------------- arguments

struct Args {
    const void* in;
    void* out;
    int64_t rows;
    int64_t stride;   // row stride in accesses (elements / access width)
    int64_t nblocks;  // logical workgroups; the grid may be smaller and loop
    int64_t diag;     // causal kernels: row i keeps columns j <= i + diag
    int64_t period;   // causal kernels: rows per matrix, i counted within its matrix; 0: one matrix
    int64_t pitch;    // bytes between row starts (any-alignment kernels)
    int nacc;         // accesses per row (cols / access width)
    int cols;         // elements per row
    float coef;       // scale * log2(e); log2(e) for the plain softmax
};

// Line shift of one row.  A 128-byte line holds 8 accesses of 16 bytes.  With
// the shift s = (address of the row's output / 16) mod 8, the row kernels'
// slot p (see first_access) holds access p - s, so every store instruction
// covers whole lines and only the row's first and last lines are split with
// its neighbours.  Rows whose width is not a multiple of 128 bytes otherwise
// split a line at every instruction's 1 KiB boundary.  The row kernels take the shift as a template flag (Shift), so
// unshifted launches run code without it (computing it costs a row kernel
// whose rows all start at once about 7%); the host picks the shifted
// instantiation only when the workgroup has spare slots for every row's shift.
constexpr int kLineAccesses = 8;

template <class E, int N, bool Shift>
__device__ inline int line_shift(const void* row_out) {
    if constexpr (!Shift || N * E::kBytes != 16) {
        return 0;
    } else {
        return int((reinterpret_cast<uintptr_t>(row_out) >> 4) & (kLineAccesses - 1));
    }
}

// Columns row `row` keeps: all of them, or the columns j <= i + diag for the
// causal (scaled, masked) softmax of "Dissecting Memory Bandwidth & SRAM
// Tiling in Triton", section "Writing the Kernel in OpenAI Triton", with i the
// row's index within its score matrix (row mod period for a batch of
// matrices, row itself for one).  No sum can overflow.
template <bool Causal>
__device__ inline int kept_cols(int64_t row, const Args& a) {
    if constexpr (!Causal) {
        return a.cols;
    } else {
        const int64_t i = a.period > 0 ? row % a.period : row;
        if (a.diag >= a.cols) return a.cols;
        if (a.diag < -i) return 0;
        const int64_t k = i + a.diag + 1;
        return k > a.cols ? a.cols : int(k);
    }
}

// Load access `idx` of a row into f, or -inf where the row has nothing to
// give: before its start (a line-shifted slot), past its end, or (causal)
// past its kept columns.  A causal access
// wholly past the kept columns is not read at all; the one that straddles
// them is read and its masked elements set to -inf.
template <class E, int N, bool Causal, bool Keep = false>
__device__ inline void load_access(const typename Access<E, N>::raw* p, int idx, int nacc, int kept, float* f) {
    if constexpr (!Causal) {
        if (idx >= 0 && idx < nacc) {
            load_elems<E, N, Keep>(p, f);
        } else {
#pragma unroll
            for (int e = 0; e < N; ++e) f[e] = -INFINITY;
        }
    } else {
        const int first = idx * N;
        if (idx >= 0 && first < kept) {
            load_elems<E, N, Keep>(p, f);
            if (first + N > kept) {
#pragma unroll
                for (int e = 0; e < N; ++e)
                    if (first + e >= kept) f[e] = -INFINITY;
            }
        } else {
#pragma unroll
            for (int e = 0; e < N; ++e) f[e] = -INFINITY;
        }
    }
}

// ------------------------------------------------ rows at any element offset
//
// When a row's start is not on a 16-byte boundary (a width that is not a
// multiple of 16 bytes, an odd row pitch, a pointer inside a chunk), the
// any-alignment kernels (Any = true) still move it in aligned 16-byte
// accesses: the chunks that hold any of its elements, counted from the chunk
// holding its first element, at chunk-relative element index lo.  The row
// covers chunk-relative elements [lo, lo + cols).  A chunk is read whole: it
// lies in one page with elements of the row, so the neighbouring rows' bytes
// it also holds are safe to read, and they are masked to -inf.  It is
// written whole when all its elements are the row's, element by element in
// the (at most two) chunks it shares with the neighbouring rows, so those
// rows' bytes are never written.  Input and output sit at the same offset in
// their chunks (the host checks), so one lo serves both.
template <class E, int N>
struct RowPos {
    const typename Access<E, N>::raw* in;
    typename Access<E, N>::raw* out;
    int lo;  // chunk-relative index of the row's first element (0 for aligned rows)
};

template <class E, int N, bool Any>
__device__ inline RowPos<E, N> row_pos(const Args& a, int64_t row) {
    typedef typename Access<E, N>::raw raw;
    if constexpr (!Any) {
        return {static_cast<const raw*>(a.in) + row * a.stride, static_cast<raw*>(a.out) + row * a.stride, 0};
    } else {
        const uintptr_t off = uintptr_t(row) * uintptr_t(a.pitch);
        const uintptr_t ia = reinterpret_cast<uintptr_t>(a.in) + off;
        const uintptr_t sub = ia & 15;
        return {reinterpret_cast<const raw*>(ia - sub),
                reinterpret_cast<raw*>(reinterpret_cast<uintptr_t>(a.out) + off - sub), int(sub) / E::kBytes};
    }
}

// Chunks a row touches: the aligned kernels' accesses per row, or (Any) the
// chunks over [lo, lo + cols).
template <class E, int N, bool Any>
__device__ inline int row_chunks(const Args& a, int lo) {
    if constexpr (!Any) return a.nacc;
    else return (lo + a.cols + N - 1) / N;
}

// Load chunk `idx` of an any-alignment row whose loaded elements are [lo, hi)
// (hi = lo + kept columns); a chunk holding none of them is not read, and f
// is then left as it was.  mask_any, run once every access of the row is
// loaded, sets what lies outside [lo, hi) to -inf: masking right after each
// load would make each load wait for the one before.
template <class E, int N, bool Keep = false>
__device__ inline void load_any(const typename Access<E, N>::raw* p, int idx, int lo, int hi, float* f) {
    const int first = idx * N;
    if (idx >= 0 && first < hi && first + N > lo) load_elems<E, N, Keep>(p, f);
}

template <int N>
__device__ inline void mask_any(int idx, int lo, int hi, float* f) {
    const int first = idx * N;
    if (first >= lo && first + N <= hi) return;  // the whole chunk is the row's: most lanes
#pragma unroll
    for (int e = 0; e < N; ++e) f[e] = first + e >= lo && first + e < hi ? f[e] : -INFINITY;
}

// Store the elements of chunk `idx` that lie in [lo, hi) (hi = lo + cols).
template <class E, int N>
__device__ inline void store_any(typename Access<E, N>::raw* q, int idx, int lo, int hi, const float* f) {
    const int first = idx * N;
    if (idx < 0 || first >= hi || first + N <= lo) return;
    if (first >= lo && first + N <= hi) {
        store_elems<E, N>(q, f);
        return;
    }
    unsigned char* b = reinterpret_cast<unsigned char*>(q);
#pragma unroll
    for (int e = 0; e < N; ++e)
        if (first + e >= lo && first + e < hi) store_elem<E>(b + e * E::kBytes, f[e]);
}

// The load of one access of a row: load_access for aligned rows, load_any for
// the rest (its loaded elements [lo, lo + kept); mask_one after all loads).
template <class E, int N, bool Causal, bool Any, bool Keep = false>
__device__ inline void load_one(const typename Access<E, N>::raw* p, int idx, int nacc, int lo, int kept, float* f) {
    if constexpr (Any) load_any<E, N, Keep>(p, idx, lo, lo + kept, f);
    else load_access<E, N, Causal, Keep>(p, idx, nacc, kept, f);
}

template <int N, bool Any>
__device__ inline void mask_one(int idx, int lo, int kept, float* f) {
    if constexpr (Any) mask_any<N>(idx, lo, lo + kept, f);
}

// ------------------------------------------------------------ packed kernel
//
// Lane l of a group of L lanes owns accesses l, l + L, l + 2L, ... of its row,
// so one load instruction of a wave reads 64 consecutive 16-byte chunks: the
// rows of a group are adjacent when the row stride equals the width.
template <class E, int N, int L, int V, int G, bool Causal, bool Any = false>
__global__ void __launch_bounds__(256) softmax_packed(Args a) {
    typedef typename Access<E, N>::raw raw;
    constexpr int kRowsPerGroup = kWave / L;
    constexpr int kRowsPerWave = kRowsPerGroup * G;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int waves = blockDim.x / kWave;
    const int sub = lane / L;
    const int l = lane % L;

    for (int64_t b = blockIdx.x; b < a.nblocks; b += gridDim.x) {
        const int64_t row0 = (b * waves + wave) * kRowsPerWave + sub;
        float x[G][V][N];
        RowPos<E, N> pos[G];  // (aligned rows: recomputed at the store)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t row = row0 + g * kRowsPerGroup;
            const bool live = row < a.rows;
            const int kept = live ? kept_cols<Causal>(row, a) : 0;
            pos[g] = row_pos<E, N, Any>(a, row);  // a row past the last is never dereferenced
            const raw* p = pos[g].in + l;
#pragma unroll
            for (int v = 0; v < V; ++v)
                load_one<E, N, Causal, Any>(p + v * L, v * L + l, live ? a.nacc : 0, pos[g].lo, kept, x[g][v]);
        }
        if constexpr (Any) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int64_t row = row0 + g * kRowsPerGroup;
                const int kept = row < a.rows ? kept_cols<Causal>(row, a) : 0;
#pragma unroll
                for (int v = 0; v < V; ++v) mask_one<N, Any>(v * L + l, pos[g].lo, kept, x[g][v]);
            }
        }
        float mx[G], r[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float m = x[g][0][0];
#pragma unroll
            for (int v = 0; v < V; ++v)
#pragma unroll
                for (int e = 0; e < N; ++e) m = fmaxf(m, x[g][v][e]);
            mx[g] = group_reduce<L, OpMax>(m);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            rebase_large_max<V * N>(&x[g][0][0], mx[g], a.coef);
            const float s = exp_and_sum<V * N>(&x[g][0][0], mx[g], a.coef);
            r[g] = recip_sum(group_reduce<L, OpSum>(s));
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t row = row0 + g * kRowsPerGroup;
            raw* p = (Any ? pos[g].out : static_cast<raw*>(a.out) + row * a.stride) + l;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                if constexpr (Any) {
                    if (row < a.rows) {
#pragma unroll
                        for (int e = 0; e < N; ++e) x[g][v][e] *= r[g];
                        store_any<E, N>(p + v * L, v * L + l, pos[g].lo, pos[g].lo + a.cols, x[g][v]);
                    }
                } else if (row < a.rows && v * L + l < a.nacc) {
#pragma unroll
                    for (int e = 0; e < N; ++e) x[g][v][e] *= r[g];
                    store_elems<E, N>(p + v * L, x[g][v]);
                }
            }
        }
    }
}

// --------------------------------------------------------------- row kernel
//
// One workgroup of W waves per row.  Wave w owns a contiguous run of 64 V
// accesses, its lane l accesses 64 V w + l, 64 V w + l + 64, ..., less the
// row's line shift (see line_shift): each load or store instruction of a
// wave covers 1 KiB, and a wave's instructions walk its run in order.  (The
// same kernels with thread t owning accesses t, t + 64 W, ... ran 1.9% slower
// on 8192 x 4096 fp16 and on 16384-column fp32 rows, and within 1% elsewhere.)
// The row stays in registers between the max, the exponentials and the
// store.  Two barriers per row: after the per-wave maxima reach LDS and after
// the per-wave sums do (separate slots, so no third barrier guards reuse).

// First access of thread t: 64 V (t / 64) + t % 64, less the line shift s.
template <int V>
__device__ inline int first_access(int t, int s) {
    return (t / kWave) * (V * kWave) + (t % kWave) - s;
}

// Thread loads accesses i0, i0 + 64, ..., i0 + 64 (V - 1) of the row (i0 from
// first_access); p addresses access i0.
template <class E, int N, int W, int V, bool Causal, bool Any = false>
__device__ inline void load_row(const typename Access<E, N>::raw* p, int i0, int nacc, int lo, int kept,
                                float (&x)[V][N]) {
#pragma unroll
    for (int v = 0; v < V; ++v) load_one<E, N, Causal, Any>(p + v * kWave, v * kWave + i0, nacc, lo, kept, x[v]);
#pragma unroll
    for (int v = 0; v < V; ++v) mask_one<N, Any>(v * kWave + i0, lo, kept, x[v]);
}

// Max, exponentials, sum and the normalised store of one row held in x.
// red_max / red_sum hold one float per wave.  Callers may run it for several
// rows in turn: every thread reads red_max before the second barrier and
// red_sum before the next call's first barrier, so the slots can be reused
// without a third barrier.
template <class E, int N, int W, int V, bool Any = false>
__device__ inline void finish_row(float (&x)[V][N], typename Access<E, N>::raw* q, int t, int i0, int nacc,
                                  float coef, float* red_max, float* red_sum, int lo = 0, int cols = 0) {
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    float m = x[0][0];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int e = 0; e < N; ++e) m = fmaxf(m, x[v][e]);
    m = group_reduce<kWave, OpMax>(m);
    if (W > 1) {
        if (lane == 0) red_max[wave] = m;
        __syncthreads();
        m = red_max[0];
#pragma unroll
        for (int w = 1; w < W; ++w) m = fmaxf(m, red_max[w]);
    }

    rebase_large_max<V * N>(&x[0][0], m, coef);
    float s = exp_and_sum<V * N>(&x[0][0], m, coef);
    s = group_reduce<kWave, OpSum>(s);
    if (W > 1) {
        if (lane == 0) red_sum[wave] = s;
        __syncthreads();
        s = red_sum[0];
#pragma unroll
        for (int w = 1; w < W; ++w) s += red_sum[w];
    }
    const float r = recip_sum(s);

#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int idx = v * kWave + i0;
        if constexpr (Any) {
#pragma unroll
            for (int e = 0; e < N; ++e) x[v][e] *= r;
            store_any<E, N>(q + v * kWave, idx, lo, lo + cols, x[v]);
        } else if (idx >= 0 && idx < nacc) {
#pragma unroll
            for (int e = 0; e < N; ++e) x[v][e] *= r;
            store_elems<E, N>(q + v * kWave, x[v]);
        }
    }
}

template <class E, int N, int W, int V, bool Causal, bool Shift = false, bool Any = false>
__global__ void __launch_bounds__(W * kWave) softmax_row(Args a) {
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    const int t = threadIdx.x;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        float x[V][N];
        const RowPos<E, N> pos = row_pos<E, N, Any>(a, row);
        const int i0 = first_access<V>(t, line_shift<E, N, Shift>(pos.out));
        load_row<E, N, W, V, Causal, Any>(pos.in + i0, i0, a.nacc, pos.lo, kept_cols<Causal>(row, a), x);
        finish_row<E, N, W, V, Any>(x, pos.out + i0, t, i0, a.nacc, a.coef, red_max, red_sum, pos.lo, a.cols);
    }
}

// ----------------------------------------------------- prefetching row kernel
//
// The same per-row work, but each workgroup stays resident and walks rows
// blockIdx.x, blockIdx.x + gridDim.x, ...; the next row's loads are issued
// before the current row is reduced, so its HBM reads overlap the current
// row's reductions, exponentials and stores.  The grid is sized to the
// number of workgroups the chip holds at once.
template <class E, int N, int W, int V, bool Causal, bool Shift = false, bool Any = false>
__global__ void __launch_bounds__(W * kWave) softmax_row_pf(Args a) {
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    const int t = threadIdx.x;
    int64_t row = blockIdx.x;
    if (row >= a.rows) return;  // uniform per workgroup: no barrier is skipped by part of it
    float nx[V][N];
    RowPos<E, N> npos = row_pos<E, N, Any>(a, row);
    int ni0 = first_access<V>(t, line_shift<E, N, Shift>(npos.out));
    load_row<E, N, W, V, Causal, Any>(npos.in + ni0, ni0, a.nacc, npos.lo, kept_cols<Causal>(row, a), nx);
    for (; row < a.rows; row += gridDim.x) {
        float x[V][N];
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int e = 0; e < N; ++e) x[v][e] = nx[v][e];
        const int i0 = ni0;
        const RowPos<E, N> pos = npos;
        const int64_t next = row + gridDim.x;
        if (next < a.rows) {
            npos = row_pos<E, N, Any>(a, next);
            ni0 = first_access<V>(t, line_shift<E, N, Shift>(npos.out));
            load_row<E, N, W, V, Causal, Any>(npos.in + ni0, ni0, a.nacc, npos.lo, kept_cols<Causal>(next, a), nx);
        }
        finish_row<E, N, W, V, Any>(x, pos.out + i0, t, i0, a.nacc, a.coef, red_max, red_sum, pos.lo, a.cols);
    }
}

// ------------------------------------------ 16-bit rows held as stored values
//
// For 16-bit rows wider than the row kernel's registers hold once widened
// (eight floats per 16-byte access): the same one workgroup per row, one read
// and one write, but each lane keeps its accesses as loaded, four registers
// each, and widens them again for every step; each exponential is computed
// twice, once for the sum and once for the output, where the online kernel
// would read the row twice.  Same frame, same order of operations as the row
// kernel, so the same bits wherever both take a row.
//
// A lane slot outside the accesses that hold the row's loaded elements (past
// its end or a causal row's kept columns, or before its start in a
// line-shifted launch) loads the nearest such access instead of nothing, so
// every load goes straight into the registers that keep it, and each step
// leaves such slots out: the max skips them and the sum keeps its value, as
// the row kernel's -inf entries (exponential +0) leave it.  Causal and
// any-offset rows mask their boundary accesses as the row kernel does.
//
// An empty asm statement that takes the stored values and gives them back
// comes before the sum and before the output: the compiler must then widen
// them afresh, instead of keeping an earlier step's widened values alive,
// which would take the registers this kernel exists to save.
template <int V>
__device__ inline void fresh(u32x4 (&xr)[V]) {
#pragma unroll
    for (int v = 0; v < V; ++v) asm volatile("" : "+v"(xr[v]));
}

template <class E>
__device__ inline void widen_access(u32x4 r, float* f) {
    widen_dword<E>(r.x, f);
    widen_dword<E>(r.y, f + 2);
    widen_dword<E>(r.z, f + 4);
    widen_dword<E>(r.w, f + 6);
}

template <class E> __device__ inline unsigned short neg_inf_half();
template <> __device__ inline unsigned short neg_inf_half<F16>() { return 0xFC00u; }
template <> __device__ inline unsigned short neg_inf_half<BF16>() { return 0xFF80u; }

// Causal and any-offset rows: the stored values outside the row's loaded
// elements [lo, hi) of access idx -- past a causal row's kept columns, or the
// neighbouring rows' elements in a shared chunk -- become -inf in place, once,
// so that every later step reads the row as the row kernel's masked loads
// leave it.  Only boundary accesses, and the slots outside the row, change.
template <class E>
__device__ inline void mask_stored(u32x4& r, int idx, int lo, int hi) {
    const int first = idx * 8;
    if (first >= lo && first + 8 <= hi) return;
    unsigned w[4] = {r.x, r.y, r.z, r.w};
    const unsigned ninf = neg_inf_half<E>();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        if (first + e < lo || first + e >= hi) {
            const int sh = 16 * (e & 1);
            w[e >> 1] = (w[e >> 1] & ~(0xFFFFu << sh)) | (ninf << sh);
        }
    }
    r = u32x4{w[0], w[1], w[2], w[3]};
}

// The row's exponentials in frame fr added to s in the row kernel's order,
// each entry first less `sub`: the max for rows rebased as in
// rebase_large_max, else +0, which leaves every entry as it is.  Accesses
// outside [0, nread) keep s as it is, as the row kernel's -inf entries do.
template <class E, int V>
__device__ inline float row16_sum(const u32x4 (&xr)[V], int i0, int nread, float sub, float coef, float fr) {
    float s = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int idx = v * kWave + i0;
        float f[8];
        widen_access<E>(xr[v], f);
        float t = s;
#pragma unroll
        for (int e = 0; e < 8; ++e) t += exp_in_frame(f[e] - sub, coef, fr);
        s = idx >= 0 && idx < nread ? t : s;
    }
    return s;
}

// The normalised output of accesses [0, nstore) of the row (any-offset rows:
// only its own elements, see store_any).
template <class E, int V, bool Any>
__device__ inline void row16_store(const u32x4 (&xr)[V], u32x4* q, int i0, int nstore, int lo, int cols, float sub,
                                   float coef, float fr, float r) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
        const int idx = v * kWave + i0;
        if (idx >= 0 && idx < nstore) {
            float f[8];
            widen_access<E>(xr[v], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = exp_in_frame(f[e] - sub, coef, fr) * r;
            if constexpr (Any) store_any<E, 8>(q + v * kWave, idx, lo, lo + cols, f);
            else store_elems<E, 8>(q + v * kWave, f);
        }
    }
}

template <class E, int W, int V, bool Causal, bool Shift = false, bool Any = false>
__global__ void __launch_bounds__(W * kWave) softmax_row16(Args a) {
    static_assert(E::kBytes == 2, "16-bit types only");
    constexpr bool kMasked = Causal || Any;
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    const float coef = a.coef;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const RowPos<E, 8> pos = row_pos<E, 8, Any>(a, row);
        const int lo = pos.lo;
        const int hi = lo + kept_cols<Causal>(row, a);  // the row's loaded elements are [lo, hi)
        const int nread = kMasked ? (hi + 7) / 8 : a.nacc;  // accesses holding any of them
        const int nstore = row_chunks<E, 8, Any>(a, lo);    // accesses the output covers
        int i0 = first_access<V>(t, line_shift<E, 8, Shift>(pos.out));
        // taken per row: per-access offsets and masks hoisted out of the row
        // loop would hold registers through all of it
        asm volatile("" : "+v"(i0));
        u32x4 xr[V];
        const int last = nread > 0 ? nread - 1 : 0;  // a row's first access always lies within it
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int idx = v * kWave + i0;
            xr[v] = ld<true>(pos.in + (idx < 0 ? 0 : idx < last ? idx : last));
        }
        if constexpr (kMasked) {
#pragma unroll
            for (int v = 0; v < V; ++v) mask_stored<E>(xr[v], v * kWave + i0, lo, hi);
        }
        float m = -INFINITY;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int idx = v * kWave + i0;
            float f[8];
            widen_access<E>(xr[v], f);
            float cm = f[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) cm = fmaxf(cm, f[e]);
            m = idx >= 0 && idx < nread ? fmaxf(m, cm) : m;
        }
        m = group_reduce<kWave, OpMax>(m);
        if (W > 1) {
            if (lane == 0) red_max[wave] = m;
            __syncthreads();
            m = red_max[0];
#pragma unroll
            for (int w = 1; w < W; ++w) m = fmaxf(m, red_max[w]);
        }
        const bool rebase = !frame_small(m, coef);  // m is the same in every lane
        const float sub = rebase ? m : 0.0f;
        const float fr = frame_of(rebase ? 0.0f : m, coef);
        fresh<V>(xr);
        float s = row16_sum<E, V>(xr, i0, nread, sub, coef, fr);
        s = group_reduce<kWave, OpSum>(s);
        if (W > 1) {
            if (lane == 0) red_sum[wave] = s;
            __syncthreads();
            s = red_sum[0];
#pragma unroll
            for (int w = 1; w < W; ++w) s += red_sum[w];
        }
        const float r = recip_sum(s);
        fresh<V>(xr);
        row16_store<E, V, Any>(xr, pos.out + i0, i0, nstore, lo, a.cols, sub, coef, fr, r);
    }
}

// ------------------------------------------------------------ online kernel
//
// One workgroup of W waves per row of any width.  Pass 1 walks the row in
// chunks of V accesses per thread; per chunk each lane takes the chunk max,
// rescales its running sum to the new max once (not once per element), and
// adds the chunk's exponentials.  The per-lane (max, sum) pairs are merged
// across the wave and then across waves through LDS.  Pass 2 re-reads the
// row and writes e^(x - m) / sum.  Traffic: two reads and one write per
// element (the second read may hit L2 or the Infinity Cache); a causal row
// reads only its kept columns, twice.
//
// Exponentials here are 2^((x - m) c), two operations: each lane's sum is
// relative to that lane's own max, and the subtraction keeps the terms of
// different lanes and both passes consistent without a shared frame.
template <class E, int N, int W, int V, bool Causal, bool Any = false>
__global__ void __launch_bounds__(W * kWave) softmax_online(Args a) {
    typedef typename Access<E, N>::raw raw;
    constexpr int kThreads = W * kWave;
    constexpr int kChunk = kThreads * V;
    __shared__ float red_m[W];
    __shared__ float red_s[W];
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    const float coef = a.coef;

    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        const RowPos<E, N> pos = row_pos<E, N, Any>(a, row);
        // Slot i of a chunk holds access i - sh (the line shift of the row
        // kernels): each wave's 64 accesses then cover whole 128-byte lines of
        // the output, where a row starting inside a line would split one at
        // every wave.  Slots before the row's first access stay empty.
        const int sh = line_shift<E, N, true>(pos.out);
        const int t0 = t - sh;  // this thread's access in chunk 0
        const raw* p = pos.in + t0;
        const int kept = kept_cols<Causal>(row, a);
        // accesses that hold at least one kept column
        const int nread = Causal || Any ? (pos.lo + kept + N - 1) / N : a.nacc;
        const int nacc = row_chunks<E, N, Any>(a, pos.lo);
        float lm = -INFINITY;  // lane running max; -inf: nothing finite seen yet
        float ls = 0.0f;       // lane sum of e^(c (x - lm))
        for (int c = 0; c < nread + sh; c += kChunk) {
            float x[V][N];
#pragma unroll
            for (int v = 0; v < V; ++v)
                load_one<E, N, Causal, Any, true>(p + c + v * kThreads, c + v * kThreads + t0, a.nacc, pos.lo, kept,
                                                  x[v]);
#pragma unroll
            for (int v = 0; v < V; ++v) mask_one<N, Any>(c + v * kThreads + t0, pos.lo, kept, x[v]);
            float cm = x[0][0];
#pragma unroll
            for (int v = 0; v < V; ++v)
#pragma unroll
                for (int e = 0; e < N; ++e) cm = fmaxf(cm, x[v][e]);
            if (cm == -INFINITY) continue;  // nothing finite in this chunk for this lane
            if (cm > lm) {
                ls *= exp_diff(lm - cm, coef);  // lm = -inf: 0 * 0
                lm = cm;
            }
            float s = 0.0f;
#pragma unroll
            for (int v = 0; v < V; ++v)
#pragma unroll
                for (int e = 0; e < N; ++e) s += exp_diff(x[v][e] - lm, coef);
            ls += s;
        }
        wave_reduce_pair(lm, ls, coef);
        if (lane == 0) {
            red_m[wave] = lm;
            red_s[wave] = ls;
        }
        __syncthreads();
        lm = red_m[0];
        ls = red_s[0];
#pragma unroll
        for (int w = 1; w < W; ++w) merge_pair(lm, ls, red_m[w], red_s[w], coef);
        const float m = lm == -INFINITY ? 0.0f : lm;  // all -inf row: every term exp(-inf) = 0
        const float r = recip_sum(ls);

        raw* q = pos.out + t0;
        for (int c = 0; c < nacc + sh; c += kChunk) {
            float x[V][N];
#pragma unroll
            for (int v = 0; v < V; ++v)
                load_one<E, N, Causal, Any>(p + c + v * kThreads, c + v * kThreads + t0, a.nacc, pos.lo, kept, x[v]);
#pragma unroll
            for (int v = 0; v < V; ++v) mask_one<N, Any>(c + v * kThreads + t0, pos.lo, kept, x[v]);
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int idx = c + v * kThreads + t0;
                if constexpr (Any) {
#pragma unroll
                    for (int e = 0; e < N; ++e) x[v][e] = exp_diff(x[v][e] - m, coef) * r;
                    store_any<E, N>(q + c + v * kThreads, idx, pos.lo, pos.lo + a.cols, x[v]);
                } else if (idx >= 0 && idx < a.nacc) {
#pragma unroll
                    for (int e = 0; e < N; ++e) x[v][e] = exp_diff(x[v][e] - m, coef) * r;
                    store_elems<E, N>(q + c + v * kThreads, x[v]);
                }
            }
        }
        __syncthreads();  // red_m / red_s are rewritten for the next row
    }
}

// ---------------------------------------------------------- split-row kernels
//
// For few, wide rows: one workgroup per row leaves most of the chip idle, so
// each row is cut into tiles of W*64*V accesses and every tile gets its own
// workgroup -- the "two passes" answer to a reduction that spans blocks ("Kernel
// Fusion", section "What fusion cannot fix"), with the tiles' partial results
// combined by the online-softmax merge ("Dissecting Memory Bandwidth & SRAM
// Tiling in Triton", section "The Mathematical Remedy: Online Softmax
// Tiling").  Kernel 1 writes each tile's (max, sum) to a workspace; kernel 2
// has every workgroup of a row merge that row's pairs in one fixed order (so
// all of them reach the same bits), re-read its tile and write it normalised.
// Traffic: two reads and one write per element; kernel 1 reads with the
// default cache policy so that kernel 2's re-read can hit L2 or the Infinity
// Cache.  No workgroup waits for another, so the grid may be any size.
//
// Rows of many tiles would have every workgroup of kernel 2 read all of the
// row's pairs (tiles^2 reads per row), so for them a kernel launched between
// the two, softmax_split_merge, merges each row's pairs once, in the same
// fixed order, and writes the merged pair back to every tile's entry; kernel 2
// (Merged = true) then reads only its own tile's entry.  The bits are the same.
//
// With Slot = true there is no workspace: each tile's pair goes to the first
// 8 bytes of the tile's own output (every tile holds at least one 16-byte
// access), and the next 4 bytes start at zero.  This needs an output distinct
// from the input.  Rows of many tiles run the merge kernel, and kernel 2 reads
// its own tile's slot before any thread of its workgroup overwrites it.  Rows
// of few tiles skip it (Slot, not Merged): every workgroup of kernel 2 merges
// the row's pairs from the slots itself and writes its tile except the
// tile's first access, which holds the slot; then it counts itself done on
// the counter in the row's first slot, and the workgroup that counts last --
// every other one of the row has read its pairs by then -- writes the first
// access of every tile of the row.  Nothing waits for anything, and the bits
// are the same as on the other paths.
struct SplitArgs {
    const void* in;
    void* out;
    float* part;     // 2 floats (max, sum) per (row, tile), row-major; unused with Slot
    int64_t rows;
    int64_t stride;  // row stride in accesses
    int64_t work;    // rows * tiles
    int nacc;        // accesses per row
    int tiles;       // tiles per row
    float coef;      // log2(e)
};

// Where tile `tile` of row `row` keeps its (max, sum) pair: the workspace, or
// (Slot) the first 8 bytes of the tile's own output.
template <class E, int N, int W, int V, bool Slot>
__device__ inline f32x2* pair_at(const SplitArgs& a, int64_t row, int tile) {
    if constexpr (Slot) {
        typedef typename Access<E, N>::raw raw;
        raw* out = static_cast<raw*>(a.out);
        return reinterpret_cast<f32x2*>(out + row * a.stride + int64_t(tile) * (W * kWave * V));
    } else {
        return reinterpret_cast<f32x2*>(a.part + 2 * (row * a.tiles + tile));
    }
}

template <class E, int N, int W, int V, bool Slot>
__global__ void __launch_bounds__(W * kWave) softmax_split_stats(SplitArgs a) {
    typedef typename Access<E, N>::raw raw;
    constexpr int kThreads = W * kWave;
    constexpr int kTile = kThreads * V;
    __shared__ float red_m[W];
    __shared__ float red_s[W];
    const raw* in = static_cast<const raw*>(a.in);
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    for (int64_t b = blockIdx.x; b < a.work; b += gridDim.x) {
        const int64_t row = b / a.tiles;
        const int base = int(b - row * a.tiles) * kTile;
        const raw* p = in + row * a.stride + base + t;
        float x[V][N];
#pragma unroll
        for (int v = 0; v < V; ++v)
            load_access<E, N, false, true>(p + v * kThreads, base + v * kThreads + t, a.nacc, 0, x[v]);
        float m = x[0][0];
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int e = 0; e < N; ++e) m = fmaxf(m, x[v][e]);
        m = group_reduce<kWave, OpMax>(m);
        if (lane == 0) red_m[wave] = m;
        __syncthreads();
        m = red_m[0];
#pragma unroll
        for (int w = 1; w < W; ++w) m = fmaxf(m, red_m[w]);
        float s = 0.0f;
        if (m != -INFINITY) {  // uniform: m is the workgroup's
#pragma unroll
            for (int v = 0; v < V; ++v)
#pragma unroll
                for (int e = 0; e < N; ++e) s += exp_diff(x[v][e] - m, a.coef);
        }
        s = group_reduce<kWave, OpSum>(s);
        if (lane == 0) red_s[wave] = s;
        __syncthreads();
        if (t == 0) {
            s = red_s[0];
#pragma unroll
            for (int w = 1; w < W; ++w) s += red_s[w];
            f32x2* slot = pair_at<E, N, W, V, Slot>(a, row, int(b - row * a.tiles));
            if constexpr (Slot) {
                // the pair, then the row's counter (used in the row's first slot) at zero
                *reinterpret_cast<u32x4*>(slot) = u32x4{__builtin_bit_cast(unsigned, m),
                                                        __builtin_bit_cast(unsigned, s), 0u, 0u};
            } else {
                *slot = f32x2{m, s};
            }
        }
        __syncthreads();  // red_m / red_s are rewritten for the next tile
    }
}

// Merge row `row`'s tile pairs in one fixed order: thread t takes tiles t,
// t + 64W, ... in order (loading eight at a time, so that a row of many tiles
// costs few round trips), then the wave and the workgroup reductions.  Every
// caller merges in this order, so all of them reach the same bits.  Every
// thread ends with the row's pair; red_m / red_s stay in use until the
// caller's next barrier.
template <class E, int N, int W, int V, bool Slot>
__device__ inline void merge_row(const SplitArgs& a, int64_t row, float* red_m, float* red_s, float& m, float& s) {
    constexpr int kThreads = W * kWave;
    constexpr int kBatch = 8;
    const int t = threadIdx.x;
    const int lane = t & (kWave - 1);
    const int wave = t / kWave;
    m = -INFINITY;
    s = 0.0f;
    int j = t;
    for (; j + (kBatch - 1) * kThreads < a.tiles; j += kBatch * kThreads) {
        f32x2 pr[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) pr[u] = *pair_at<E, N, W, V, Slot>(a, row, j + u * kThreads);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) merge_pair(m, s, pr[u].x, pr[u].y, a.coef);
    }
    for (; j < a.tiles; j += kThreads) {
        const f32x2 pr = *pair_at<E, N, W, V, Slot>(a, row, j);
        merge_pair(m, s, pr.x, pr.y, a.coef);
    }
    wave_reduce_pair(m, s, a.coef);
    if (lane == 0) {
        red_m[wave] = m;
        red_s[wave] = s;
    }
    __syncthreads();
    m = red_m[0];
    s = red_s[0];
#pragma unroll
    for (int w = 1; w < W; ++w) merge_pair(m, s, red_m[w], red_s[w], a.coef);
}

// Merge each row's tile pairs once (merge_row) and write the merged pair back
// to every tile's entry of the row.  Each entry is read, and later written,
// by the same thread.
template <class E, int N, int W, int V, bool Slot>
__global__ void __launch_bounds__(W * kWave) softmax_split_merge(SplitArgs a) {
    constexpr int kThreads = W * kWave;
    __shared__ float red_m[W];
    __shared__ float red_s[W];
    const int t = threadIdx.x;
    for (int64_t row = blockIdx.x; row < a.rows; row += gridDim.x) {
        float m, s;
        merge_row<E, N, W, V, Slot>(a, row, red_m, red_s, m, s);
        const f32x2 merged = {m, s};
        for (int j = t; j < a.tiles; j += kThreads) *pair_at<E, N, W, V, Slot>(a, row, j) = merged;
        __syncthreads();  // red_m / red_s are rewritten for the next row
    }
}

template <class E, int N, int W, int V, bool Slot, bool Merged>
__global__ void __launch_bounds__(W * kWave) softmax_split_norm(SplitArgs a) {
    typedef typename Access<E, N>::raw raw;
    constexpr bool kDirect = Slot && !Merged;  // few tiles: the slots merged here, last workgroup finishes
    constexpr int kThreads = W * kWave;
    constexpr int kTile = kThreads * V;
    __shared__ float red_m[W];
    __shared__ float red_s[W];
    const raw* in = static_cast<const raw*>(a.in);
    raw* out = static_cast<raw*>(a.out);
    const int t = threadIdx.x;
    for (int64_t b = blockIdx.x; b < a.work; b += gridDim.x) {
        const int64_t row = b / a.tiles;
        const int base = int(b - row * a.tiles) * kTile;
        const raw* p = in + row * a.stride + base + t;
        float x[V][N];
#pragma unroll
        for (int v = 0; v < V; ++v) load_access<E, N, false>(p + v * kThreads, base + v * kThreads + t, a.nacc, 0, x[v]);
        float m, s;
        if constexpr (Merged) {
            // the row's merged pair, already in this tile's entry
            const f32x2 pr = *pair_at<E, N, W, V, Slot>(a, row, int(b - row * a.tiles));
            m = pr.x;
            s = pr.y;
            if constexpr (Slot) __syncthreads();  // all have read the slot before the tile's first access is rewritten
        } else {
            merge_row<E, N, W, V, Slot>(a, row, red_m, red_s, m, s);
        }
        const float mu = m == -INFINITY ? 0.0f : m;  // all -inf row: every term exp(-inf) = 0
        const float r = recip_sum(s);
        raw* q = out + row * a.stride + base + t;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            // (kDirect: the tile's first access holds the slot, written last)
            if (base + v * kThreads + t < a.nacc && !(kDirect && v == 0 && t == 0)) {
#pragma unroll
                for (int e = 0; e < N; ++e) x[v][e] = exp_diff(x[v][e] - mu, a.coef) * r;
                store_elems<E, N>(q + v * kThreads, x[v]);
            }
        }
        if constexpr (kDirect) {
            // merge_row's reads of the slots are complete in every thread
            // (their values went into its reduction, which ends at a
            // barrier); count this tile done.  The count needs no release or
            // acquire: the slots were written by the previous kernel, and the
            // last workgroup's stores depend on the count's result.  (An
            // agent-scope release would write back this XCD's L2 for every
            // tile.)
            __shared__ int last;
            if (t == 0) {
                unsigned* counter = reinterpret_cast<unsigned*>(pair_at<E, N, W, V, Slot>(a, row, 0)) + 2;
                const unsigned done =
                    __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last = done == unsigned(a.tiles - 1);
            }
            __syncthreads();
            if (last) {
                // every workgroup of the row has read its pairs: write the
                // first access of each tile (slot and counter included)
                for (int j = t; j < a.tiles; j += kThreads) {
                    const int64_t at = row * a.stride + int64_t(j) * kTile;
                    float f[N];
                    load_access<E, N, false>(in + at, j * kTile, a.nacc, 0, f);
#pragma unroll
                    for (int e = 0; e < N; ++e) f[e] = exp_diff(f[e] - mu, a.coef) * r;
                    store_elems<E, N>(out + at, f);
                }
            }
        }
        __syncthreads();  // red_m / red_s (and `last`) are rewritten for the next tile
    }
}

// ------------------------------------------------------------- copy kernel
//
// Plain 16-byte copy with the same non-temporal hints, U accesses per thread in
// flight: the achievable read-once/write-once bandwidth that a finished
// softmax is compared with.
template <int U>
__global__ void __launch_bounds__(256) copy16(const u32x4* src, u32x4* dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * U;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x; base < n; base += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + (int64_t)u * blockDim.x < n) v[u] = ld<true>(src + base + (int64_t)u * blockDim.x);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + (int64_t)u * blockDim.x < n) st<true>(dst + base + (int64_t)u * blockDim.x, v[u]);
    }
}

// Copy in contiguous per-workgroup chunks of W * 64 * V 16-byte accesses,
// shaped like the row kernels without their arithmetic: wave w loads its run
// of 64 V accesses (lane l: accesses 64 V w + l + 64 v), the workgroup waits
// at a barrier, then stores them.  Timing the chunk sizes of the row kernels
// this way separates the cost of the access pattern from the softmax's own.
template <int W, int V>
__global__ void __launch_bounds__(W * kWave) chunk_copy16(const u32x4* src, u32x4* dst, int64_t nchunks) {
    const int t = threadIdx.x;
    const int64_t wave_run = int64_t(t / kWave) * (kWave * V) + (t % kWave);
    for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
        const int64_t base = c * (W * kWave * V) + wave_run;
        u32x4 x[V];
#pragma unroll
        for (int v = 0; v < V; ++v) x[v] = ld<true>(src + base + v * kWave);
        __syncthreads();
#pragma unroll
        for (int v = 0; v < V; ++v) st<true>(dst + base + v * kWave, x[v]);
    }
}

// Read-only and write-only streams of the same shape: the two halves of the
// copy, to show how much of a copy's time each direction costs at a size.
// The read kernel folds its data into one word and stores it only if it equals
// `never`, a value the caller picks so that the store does not happen; the
// loads cannot be dropped.
template <int U>
__global__ void __launch_bounds__(256) read16(const u32x4* src, unsigned* sink, int64_t n, unsigned never) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * U;
    unsigned acc = 0;
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x; base < n; base += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v[u] = u32x4{0, 0, 0, 0};
            if (base + (int64_t)u * blockDim.x < n) v[u] = ld<true>(src + base + (int64_t)u * blockDim.x);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == never) sink[0] = acc;
}

template <int U>
__global__ void __launch_bounds__(256) write16(u32x4* dst, int64_t n, unsigned value) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x * U;
    const u32x4 v = {value, value, value, value};
    for (int64_t base = (int64_t)blockIdx.x * blockDim.x * U + threadIdx.x; base < n; base += stride) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + (int64_t)u * blockDim.x < n) st<true>(dst + base + (int64_t)u * blockDim.x, v);
    }
}

}  // namespace rws
