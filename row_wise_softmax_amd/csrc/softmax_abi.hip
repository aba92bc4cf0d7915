// softmax_abi.hip -- the C ABI of include/row_wise_softmax.h: argument
// validation, the width dispatch and the launches.
//
// Dispatch by width, following the pages' two lessons on shapes: a fused
// kernel that gives each row a whole program wastes the machine on narrow rows
// (launch and scheduling costs dominate, "fused-softmax-roofline", the
// discussion of shapes where it loses), and a fixed block size starves wide
// rows of loads in flight ("GPU Kernels - Implementing and optimizing
// Softmax", sections "Results for this specific kernel" and "CUDA scaling
// threads").  So narrow rows share a wave (packed), mid-size rows get a wave
// or a workgroup that holds the row in registers (row), and rows past the
// register budget stream twice (online).
#include <hip/hip_runtime.h>

#include <atomic>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "kernel_table.hpp"
#include "row_wise_softmax.h"
#include "softmax_kernels.hpp"

namespace {

using rws::Entry;

constexpr int64_t kMaxGrid = int64_t(1) << 20;  // workgroups per launch; kernels loop past it
constexpr int64_t kMaxCols = int64_t(1) << 30;  // keeps every in-row index, chunk offset included, in int
constexpr double kLog2eD = 1.4426950408889634074;

int elem_bytes(int dtype) { return dtype == SOFTMAX_F32 ? 4 : 2; }

const Entry* table_of(int dtype, int* n) {
    switch (dtype) {
        case SOFTMAX_F32: *n = rws::kTableF32Size; return rws::kTableF32;
        case SOFTMAX_F16: *n = rws::kTableF16Size; return rws::kTableF16;
        case SOFTMAX_BF16: *n = rws::kTableBF16Size; return rws::kTableBF16;
        default: *n = 0; return nullptr;
    }
}

int total_kernels() { return rws::kTableF32Size + rws::kTableF16Size + rws::kTableBF16Size; }

// Global kernel id -> entry (ids run over the f32, f16 and bf16 tables in order).
const Entry* entry_by_id(int id) {
    if (id < 0) return nullptr;
    if (id < rws::kTableF32Size) return &rws::kTableF32[id];
    id -= rws::kTableF32Size;
    if (id < rws::kTableF16Size) return &rws::kTableF16[id];
    id -= rws::kTableF16Size;
    if (id < rws::kTableBF16Size) return &rws::kTableBF16[id];
    return nullptr;
}

int id_of(const Entry* e) {
    int base = 0;
    for (int dt = SOFTMAX_F32; dt <= SOFTMAX_BF16; ++dt) {
        int n;
        const Entry* t = table_of(dt, &n);
        if (e >= t && e < t + n) return base + int(e - t);
        base += n;
    }
    return -1;
}

// Widest row an entry holds: lanes (or threads) x accesses each x elements per
// access; an any-alignment entry gives up vec - 1 of them to the row's offset
// in its first chunk.
int64_t max_cols_of(const Entry& e) {
    if (e.variant == SOFTMAX_VARIANT_ONLINE) return -1;
    return int64_t(e.lanes) * e.vpl * e.vec - (e.any ? e.vec - 1 : 0);
}

// Whether rows of this call can take the any-alignment kernels: element-
// aligned pointers at the same offset in their 16-byte chunks, so that each
// chunk of the input row maps onto one chunk of the output row.
bool any16(const void* in, const void* out, int dtype) {
    const uintptr_t esz = uintptr_t(elem_bytes(dtype));
    return uintptr_t(in) % esz == 0 && uintptr_t(out) % esz == 0 && (uintptr_t(in) - uintptr_t(out)) % 16 == 0;
}

bool fits(const Entry& e, const void* in, const void* out, int64_t cols, int64_t row_stride, int dtype) {
    if (e.dtype != dtype) return false;
    if (e.any) {
        if (!any16(in, out, dtype)) return false;
    } else if (e.vec > 1) {
        const uintptr_t acc = uintptr_t(e.vec) * elem_bytes(dtype);
        if (uintptr_t(in) % acc || uintptr_t(out) % acc) return false;
        if ((uint64_t(row_stride) * elem_bytes(dtype)) % acc) return false;
        if (cols % e.vec) return false;
    }
    const int64_t mc = max_cols_of(e);
    return mc < 0 || cols <= mc;
}

const Entry* find(int dtype, int variant, bool causal, int vec, int lanes, int vpl, int groups, bool any = false) {
    int n;
    const Entry* t = table_of(dtype, &n);
    for (int i = 0; i < n; ++i) {
        const Entry& e = t[i];
        if (e.variant == variant && e.causal == causal && e.any == any && e.vec == vec && e.lanes == lanes &&
            e.vpl == vpl && e.groups == groups)
            return &e;
    }
    return nullptr;
}

// 16-byte accesses need 16-byte-aligned pointers, a 16-byte-multiple row
// pitch and a width that is a whole number of accesses.
bool aligned16(const void* in, const void* out, int64_t cols, int64_t row_stride, int dtype) {
    const int64_t esz = elem_bytes(dtype);
    return uintptr_t(in) % 16 == 0 && uintptr_t(out) % 16 == 0 && (row_stride * esz) % 16 == 0 &&
           (cols * esz) % 16 == 0;
}

// One round of the chip's wave slots (256 CUs x 4 SIMDs x 8 waves), and two.
constexpr int64_t kOneRoundWaves = 256 * 4 * 8;
constexpr int64_t kFewRowWaves = 2 * kOneRoundWaves;

int pow2_at_least(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// The width dispatch rule, set from the width sweep (bench.py --sweep, bf16
// and fp32, widths 32 ... 16384 at about 200 MB per tensor): up to 2048
// 16-byte accesses per row the fastest shape keeps about two loads in flight
// per lane and spreads the row over as many lanes as that takes (with a few
// measured exceptions for ragged rows of 129..255 accesses, see below);
// wider rows do best on four waves with more loads each.  `nacc` is the row length in 16-byte accesses (for
// rows at any element offset, the most chunks a row can touch).  The causal
// table, and the any-alignment entries (any = true), hold the same picks.
const Entry* pick_16byte(int dtype, bool causal, bool any, int64_t rows, int64_t nacc) {
    const int vec16 = 16 / elem_bytes(dtype);
    const Entry* e = nullptr;
    if (nacc <= 64) {
        // several rows per wave: L lanes per row, two row groups in flight
        e = find(dtype, SOFTMAX_VARIANT_PACKED, causal, vec16, pow2_at_least(nacc), 1, 2, any);
    } else if (nacc <= 128) {
        e = find(dtype, SOFTMAX_VARIANT_PACKED, causal, vec16, 64, 2, 1, any);
    } else if (nacc <= 2048) {
        // Ragged rows of 129..255 accesses take the general two-wave shape
        // below (bf16 1200 columns x 64 K rows: 5650 GB/s, against 4597 on
        // four waves of one; fp32 600 columns: 6020 against 4977 on four
        // waves of two), with three exceptions measured across 2 K-64 K
        // rows.  fp32 rows of 240 accesses or more (960 columns), from 8192
        // rows on: four waves of two, half the slots idle (1000 columns x
        // 64 K rows: 6446 against 6244).  16-bit rows of more than 250
        // accesses past 8192 rows: four waves of one, whose 512 slots hold
        // the line shift that 256 cannot (bf16 2040 columns x 64 K rows:
        // 5987 against 5532).  (16-bit jobs of few rows take four waves of
        // one by the one-round rule below.)
        if (nacc < 256) {
            int v = 0;
            if (dtype == SOFTMAX_F32) {
                if (nacc >= 240 && rows >= 8192) v = 2;
            } else if (nacc > 250 && rows > 8192) {
                v = 1;
            }
            if (v > 0) e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * 4, v, 1, any);
        }
        // otherwise one workgroup per row, two accesses per lane, up to 16
        // waves (2048 accesses, 16384 bf16 columns: 6150 GB/s on sixteen
        // waves against 5600 on four waves of eight; 8192 fp32 columns:
        // 6220 against 6117)
        const int w2 = pow2_at_least((nacc + 127) / 128);
        // A row at any offset can touch one chunk more than its width needs,
        // which past a power of two would double the waves and leave half
        // of them idle (4097 bf16 columns: 4120 GB/s on eight waves of two);
        // half the waves with three accesses each hold it instead.
        if (e == nullptr && any && w2 >= 4 && nacc <= (w2 / 2) * 64 * 3)
            e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * (w2 / 2), 3, 1, any);
        // fp32 rows that fill the two-access shape exactly (256 or 512
        // accesses), in jobs of 16384 rows or more: twice the waves, half the
        // slots idle (bench.py --past-pow2, GB/s: 2048 columns x 49152 rows
        // 6526 -> 6668, x 16384 rows 6308 -> 6366; 1024 x 49152: 6478 ->
        // 6545).  Below 16384 rows the gain is within 1% or a loss (1024
        // columns x 8192 rows: 5248 against 5177).  16-bit rows lost 10-20%
        // on twice the waves at 4 K-48 K rows (2048 bf16 columns x 49152
        // rows: 5529 against 6378, a probe), so they keep theirs.
        if (e == nullptr && !any && !causal && dtype == SOFTMAX_F32 && (nacc == 256 || nacc == 512) &&
            rows >= 16384)
            e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * 2 * w2, 2, 1, false);
        // Aligned rows just past a power of two take half the waves with
        // three accesses each too, where a scan found it faster
        // (bench.py --past-pow2: chunk counts 300..3800 at about 200 MB and
        // 50 MB per tensor, GB/s): 16-bit rows that fill at most 75% of the
        // two-access shape's slots on sixteen waves (1100 chunks, 8800 bf16
        // columns: 4819 -> 6042; 1500 chunks: 5654 -> 6022), 70% on eight
        // (520 chunks: 5260 -> 6192) or 62% on four (300 chunks: 5889 ->
        // 6185), fp32 rows that fill at most 62% of sixteen waves (1100
        // chunks, 4400 columns: 5971 -> 6451) or 53% of eight (520 chunks:
        // 6207 -> 6483).  Fuller rows keep two accesses (750 chunks, bf16:
        // 6140 against 6024 on three; fp32: 6495 against 6049), and so do jobs
        // of few rows, for the persistent twin below.
        if (e == nullptr && !any && w2 >= 4 && rows * (w2 / 2) > kFewRowWaves) {
            const int64_t slots2 = int64_t(w2) * 128;
            const bool v3 = elem_bytes(dtype) == 2
                                ? (w2 >= 16 ? nacc * 100 <= slots2 * 75
                                   : w2 == 8 ? nacc * 10 <= slots2 * 7
                                             : nacc * 100 <= slots2 * 62)
                                : (w2 >= 16 ? nacc * 100 <= slots2 * 62 : w2 == 8 && nacc * 100 <= slots2 * 53);
            if (v3) e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * (w2 / 2), 3, 1, false);
        }
        if (e == nullptr) e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * w2, 2, 1, any);
        // Few rows: when the whole job fills the chip's wave slots at most
        // twice, every workgroup of a round starts, loads and computes
        // together, and HBM idles while a round computes.  The row kernel's
        // persistent twin (same shape, grid = resident workgroups, the next
        // row's loads issued before the current row's reductions) keeps
        // loads in flight: 1-5% faster at one round or less, 2-21% at two
        // (4096 x 4096 bf16: 5044 -> 5973 GB/s; 2048 x 2048 fp32: 5080 ->
        // 5170).  From four rounds on the plain kernel is 1-7% ahead.
        // Plain aligned fp32 rows on sixteen waves keep the twin up to two
        // and a half rounds (bench.py --past-pow2, 2048 accesses: 1025 rows
        // 4844 -> 5588 GB/s, 1200 rows 4980 -> 5596; at 1400 rows the two
        // are even, 5196 against 5231).
        const int64_t few_waves =
            dtype == SOFTMAX_F32 && !causal && !any && e != nullptr && e->lanes == 64 * 16
                ? kFewRowWaves + kFewRowWaves / 4
                : kFewRowWaves;
        if (e != nullptr && rows * (e->lanes / 64) <= few_waves) {
            const Entry* pf = find(dtype, SOFTMAX_VARIANT_ROW_PF, causal, vec16, e->lanes, e->vpl, 1, any);
            if (pf != nullptr) e = pf;
        }
        // 16-bit jobs that twice the waves, one access each, still hold in
        // one round: the twin on those, for twice the rows' loads issued at
        // once (bf16, 256-2048 rows of 2048-8192 columns: 0.5-8% faster;
        // 256 x 8192: 1832 -> 1980 GB/s).  At two rounds it is 9-16% slower.
        if (e != nullptr && e->variant == SOFTMAX_VARIANT_ROW_PF && elem_bytes(dtype) == 2 && e->vpl == 2 &&
            rows * (2 * e->lanes / 64) <= kOneRoundWaves) {
            const Entry* one = find(dtype, SOFTMAX_VARIANT_ROW_PF, causal, vec16, 2 * e->lanes, 1, 1, any);
            if (one != nullptr) e = one;
        }
        // 16-bit rows of 1537..2000 accesses in jobs of 1281..3072 rows (two
        // to six rounds of sixteen-wave workgroups): eight waves of four, as
        // they are (1950 chunks x 1602 bf16 rows: 4875 -> 5289 GB/s; 1650 x
        // 1893: 4784 -> 5056).  Their persistent twin is no faster than
        // sixteen waves of two; those lead again from about 6400 rows (1950
        // x 6410: 5988 against 5889), and at 2048 chunks from 1400 rows.
        if (!any && elem_bytes(dtype) == 2 && nacc > 1536 && nacc <= 2000 && rows > 1280 && rows <= 3072) {
            const Entry* w8 = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * 8, 4, 1, false);
            if (w8 != nullptr) e = w8;
        }
        // 16-bit jobs just past the twin's two rounds: a quarter of the
        // waves with eight accesses each, plain, holds the whole job in one
        // round.  At 86 registers that shape keeps five waves per SIMD: five
        // workgroups of four waves per CU (1280 rows) or ten of two (2560).
        // Past one round it falls behind (bench.py --past-pow2, GB/s: 2048
        // accesses x 1025 rows 4523 -> 5483, x 1280 rows 4915 -> 5895, x
        // 1400 rows 4975 against 4520; 1600 accesses x 1200 rows 4541 ->
        // 5349; 1024 accesses x 2049 rows 4933 -> 5423, x 2560 rows 5180 ->
        // 5827, x 2800 rows 5328 against 4496).
        if (!any && !causal && elem_bytes(dtype) == 2) {
            const Entry* q = nullptr;
            if (nacc > 1536 && rows > 1024 && rows <= 1280)
                q = find(dtype, SOFTMAX_VARIANT_ROW, false, vec16, 64 * 4, 8, 1, false);
            else if (nacc > 768 && nacc <= 1024 && rows > 2048 && rows <= 2560)
                q = find(dtype, SOFTMAX_VARIANT_ROW, false, vec16, 64 * 2, 8, 1, false);
            if (q != nullptr) e = q;
        }
    } else if (elem_bytes(dtype) == 2) {
        // 16-bit rows past 2048 chunks (16384 columns) hold 8 values per
        // chunk, so four or eight waves of 16 accesses need 128 registers of
        // them per lane; sixteen waves do better (bf16, about 200 MB tensors:
        // 24576 columns 5670 GB/s on sixteen waves of four against 3513 on
        // four of sixteen; 32000: 5618 against 4025; 65536: 4965 on sixteen
        // of eight against 4243 on eight of sixteen).  Rows that leave more
        // than a tenth of sixteen waves of eight idle take the online kernel
        // (50304 columns: 4831 GB/s on sixteen waves of two chunks, against
        // 3509 on eight waves of sixteen).
        // Rows at any offset carry the boundary masks, which cost the
        // sixteen-wave shapes of four or more accesses their second
        // workgroup per CU; they take sixteen waves of three up to 3072
        // chunks, eight waves of eight up to 4096 (32001 bf16 columns: 5039
        // GB/s against 4326 on sixteen of four) and sixteen waves of eight
        // up to 8192 (50257 columns: 4211 against 3663 online).
        // Rows past 4096 chunks (32768 columns) keep their stored 16-bit
        // values in registers (softmax_row16, half the registers of widened
        // values), up to 24576 chunks (196608 columns; causal and any-offset
        // rows, whose masked forms would spill beyond, up to 16384): one read
        // instead of the online kernel's two.  Shapes by width from a sweep
        // at about 200 MB per tensor (bf16, GB/s, against the online kernel
        // or the widened row kernel before): eight waves of 12, 16 or 20
        // accesses up to 6144, 8192 and 10240 chunks (40960 columns: 5580
        // against 4771; 65536: 5643 against 4934; 81920: 5075 against 4488),
        // sixteen waves of 12, 16, 20 or 24 beyond (98304: 4627 against
        // 4485; 128256: 4255 against 4145, 5092 against 4694 at 4096 rows;
        // 151936: 4484 against 4256).  Any-offset rows gain 7-43% (50257
        // columns: 5038 against 4189), causal rows up to 13% (the last 2048
        // queries of a 65536-key causal matrix: 5575 against 4983).
        if (nacc > 4096) {
            struct Shape { int64_t chunks; int waves, vpl; };
            constexpr Shape kRow16[] = {{6144, 8, 12},   {8192, 8, 16},   {10240, 8, 20}, {12288, 16, 12},
                                        {16384, 16, 16}, {20480, 16, 20}, {24576, 16, 24}};
            for (const Shape& r : kRow16) {
                if (nacc <= r.chunks) {
                    e = find(dtype, SOFTMAX_VARIANT_ROW16, causal, vec16, 64 * r.waves, r.vpl, 1, any);
                    break;
                }
            }
        }
        if (e == nullptr && any) {
            if (nacc <= 3072) e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * 16, 3, 1, true);
            else if (nacc <= 4096) e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * 8, 8, 1, true);
            else if (nacc <= 8192) e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * 16, 8, 1, true);
        } else if (e == nullptr && nacc <= 4096) {
            // up to 3072 chunks sixteen waves of three (2500 chunks, 20000
            // bf16 columns: 5354 -> 5880 GB/s; 2200: 5188 -> 5674)
            if (nacc <= 3072) e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * 16, 3, 1, false);
            if (e == nullptr) e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * 16, 4, 1, false);
        } else if (e == nullptr && nacc <= 8192 && nacc * 10 >= 8192 * 9) {
            e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * 16, 8, 1, false);
        }
        if (e == nullptr) e = find(dtype, SOFTMAX_VARIANT_ONLINE, causal, vec16, 64 * 16, any ? 4 : 2, 1, any);
        if (e == nullptr) e = find(dtype, SOFTMAX_VARIANT_ONLINE, causal, vec16, 64 * 16, 4, 1, any);
    } else {
        // wider rows: four waves with more accesses each (16384 fp32
        // columns: 5825 GB/s, against 5625 on eight waves and 5613 on
        // sixteen); where the table has no such shape, 8 or 16 waves
        // Up to 3072 chunks sixteen waves of three instead (2800 chunks,
        // 11200 columns: 6063 -> 6254 GB/s; 2200: 6022 -> 6240; at 1116
        // rows 5075 -> 5340).
        if (!any && nacc <= 3072) e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * 16, 3, 1, false);
        const int v4 = pow2_at_least((nacc + 255) / 256);
        for (int w = 4; w <= 16 && e == nullptr; w *= 2) {
            const int v = v4 * 4 / w;
            if (v >= 1) e = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * w, v, 1, any);
        }
        // A row at any offset just past a power of two would leave a quarter
        // or more of that shape's slots idle: sixteen waves with as few
        // accesses each as hold it instead (16385 bf16 columns, 2049 chunks:
        // 3609 GB/s on eight waves of eight, 5183 on sixteen of three)
        if (any && (e == nullptr || nacc * 4 < int64_t(e->lanes) * e->vpl * 3) && nacc <= 8 * 1024) {
            const int v = int((nacc + 1023) / 1024);
            const Entry* w16 = find(dtype, SOFTMAX_VARIANT_ROW, causal, vec16, 64 * 16, v == 7 ? 8 : v, 1, any);
            if (w16 != nullptr) e = w16;
        }
        if (e == nullptr) e = find(dtype, SOFTMAX_VARIANT_ONLINE, causal, vec16, 64 * 16, 4, 1, any);
    }
    return e;
}

const Entry* select_entry(const void* in, const void* out, int64_t rows, int64_t cols, int64_t row_stride,
                          int dtype, bool causal) {
    const int vec16 = 16 / elem_bytes(dtype);
    if (aligned16(in, out, cols, row_stride, dtype)) {
        const Entry* e = pick_16byte(dtype, causal, false, rows, cols / vec16);
        if (e && fits(*e, in, out, cols, row_stride, dtype)) return e;
    } else if (any16(in, out, dtype)) {
        // rows at any element offset: the same rule on the chunks a row can touch
        const Entry* e = pick_16byte(dtype, causal, true, rows, (cols + 2 * vec16 - 2) / vec16);
        if (e && fits(*e, in, out, cols, row_stride, dtype)) return e;
    }
    // Pointers at different offsets in their 16-byte chunks: scalar accesses, streamed twice.
    const int w = cols <= 64 * 8 ? 1 : (cols <= 4 * 64 * 8 * 4 ? 4 : 16);
    return find(dtype, SOFTMAX_VARIANT_ONLINE, causal, 1, 64 * w, 8, 1);
}

// The plain table entry softmax_fwd_variant runs: of the entries of `variant`
// for this dtype whose lanes per row (packed) or threads per workgroup (row,
// row_pf, online) equal `block` and that take the call, the one on 16-byte
// accesses if any, then with the fewest accesses per lane, then the fewest
// row groups in flight.
const Entry* entry_for_variant(const void* in, const void* out, int64_t cols, int64_t row_stride, int dtype,
                               int variant, int block) {
    int n;
    const Entry* t = table_of(dtype, &n);
    const Entry* best = nullptr;
    for (int i = 0; i < n; ++i) {
        const Entry& e = t[i];
        if (e.causal || e.variant != variant) continue;
        if ((variant == SOFTMAX_VARIANT_PACKED ? e.lanes : e.block) != block) continue;
        if (!fits(e, in, out, cols, row_stride, dtype)) continue;
        if (best == nullptr || (e.vec > 1) > (best->vec > 1) ||
            ((e.vec > 1) == (best->vec > 1) &&
             (!e.any > !best->any ||
              (e.any == best->any &&
               (e.vpl < best->vpl || (e.vpl == best->vpl && e.groups < best->groups))))))
            best = &e;
    }
    return best;
}

// Shared validation.  Returns SOFTMAX_OK, or an error; *empty is set when
// there is nothing to launch.
int validate(const void* in, const void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
             bool* empty) {
    *empty = false;
    if (dtype != SOFTMAX_F32 && dtype != SOFTMAX_F16 && dtype != SOFTMAX_BF16) return SOFTMAX_ERR_BAD_DTYPE;
    if (rows < 0 || cols < 0) return SOFTMAX_ERR_BAD_SHAPE;
    if (rows == 0 || cols == 0) {
        *empty = true;
        return SOFTMAX_OK;
    }
    if (in == nullptr || out == nullptr) return SOFTMAX_ERR_NULL_POINTER;
    if (row_stride < cols) return SOFTMAX_ERR_BAD_SHAPE;
    if (cols > kMaxCols) return SOFTMAX_ERR_BAD_SHAPE;
    const int64_t esz = elem_bytes(dtype);
    // extent = ((rows - 1) * row_stride + cols) * esz must fit in int64.
    if (rows - 1 > (INT64_MAX / esz - cols) / row_stride) return SOFTMAX_ERR_BAD_SHAPE;
    const int64_t extent = ((rows - 1) * row_stride + cols) * esz;
    if (in != out) {
        const uintptr_t a = uintptr_t(in), b = uintptr_t(out);
        if (a < b + uint64_t(extent) && b < a + uint64_t(extent)) return SOFTMAX_ERR_OVERLAP;
    }
    return SOFTMAX_OK;
}

// The exponent coefficient scale * log2(e), rounded once to fp32; scale must
// be finite and > 0 (the max of scale * x is then scale * max x).
bool coef_of(float scale, float* coef) {
    if (!(scale > 0.0f) || isinf(scale)) return false;
    const double c = double(scale) * kLog2eD;
    if (!(c <= double(3.0e38f))) return false;
    *coef = float(c);
    return *coef > 0.0f;
}

// Workgroups of entry `e`'s kernel `fn` (its plain or its line-shifted
// instantiation, whose register counts, and so occupancy, can differ) the
// current device holds at once (occupancy per CU x CU count), cached per
// device, kernel and instantiation.  Used to size persistent grids.
constexpr int kMaxDevices = 64;
constexpr int kMaxKernels = 1024;
std::atomic<int> g_resident[kMaxDevices][2][kMaxKernels];  // 0 = not yet known

int64_t resident_workgroups(const Entry& e, const void* fn, int block) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const int id = id_of(&e);
    const int shifted = fn == e.fn ? 0 : 1;
    const bool cacheable = dev >= 0 && dev < kMaxDevices && id >= 0 && id < kMaxKernels;
    if (cacheable) {
        const int known = g_resident[dev][shifted][id].load(std::memory_order_relaxed);
        if (known > 0) return known;
    }
    int per_cu = 0, cus = 0;
    if (dev < 0 || hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu <= 0 ||
        cus <= 0) {
        (void)hipGetLastError();
        return 256 * 4;  // a safe default: the kernel loops over whatever rows remain
    }
    const int n = per_cu * cus;
    if (cacheable) g_resident[dev][shifted][id].store(n, std::memory_order_relaxed);
    return n;
}

// Whether a row-kernel launch shifts rows onto 128-byte lines (the kernels'
// line_shift): only for 16-byte accesses, only when some row starts inside a
// line, and only when the workgroup has a spare slot for every access the
// largest shift pushes past its last slot.  Row r's shift is
// (out / 16 + r * pitch / 16) mod 8, a sequence with period at most 8.
bool line_shift_fits(const Entry& e, const void* out, int64_t cols, int64_t row_stride) {
    if (e.variant != SOFTMAX_VARIANT_ROW && e.variant != SOFTMAX_VARIANT_ROW_PF && e.variant != SOFTMAX_VARIANT_ROW16)
        return false;
    const int64_t esz = elem_bytes(e.dtype);
    if (e.vec * esz != 16) return false;
    // row r's first chunk is line (out + r * pitch bytes) / 16 mod 8 of its
    // 128-byte line, which repeats with a period dividing 128 rows
    const uint64_t pitch = uint64_t(row_stride) * uint64_t(esz);
    int64_t most = 0;
    for (uint64_t r = 0; r < 128; ++r) {
        const int64_t sh = int64_t(((uintptr_t(out) + r * pitch) >> 4) & 7);
        most = sh > most ? sh : most;
    }
    const int64_t chunks = e.any ? (cols + 2 * e.vec - 2) / e.vec : cols / e.vec;
    const int64_t slots = int64_t(e.lanes) * e.vpl;
    return most > 0 && slots >= chunks + most;
}

int launch(const Entry& e, const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride, float coef,
           int64_t diag, hipStream_t stream, int64_t period = 0) {
    rws::Args a;
    a.in = in;
    a.out = out;
    a.rows = rows;
    a.stride = row_stride / e.vec;
    a.diag = diag;
    a.period = period;
    a.pitch = row_stride * elem_bytes(e.dtype);
    a.nacc = int(e.any ? (cols + 2 * e.vec - 2) / e.vec : cols / e.vec);
    a.cols = int(cols);
    a.coef = coef;
    const void* fn = (e.fn_shifted != nullptr && line_shift_fits(e, out, cols, row_stride)) ? e.fn_shifted : e.fn;
    int block;
    if (e.variant == SOFTMAX_VARIANT_PACKED) {
        const int64_t rows_per_wave = int64_t(64 / e.lanes) * e.groups;
        const int64_t waves = (rows + rows_per_wave - 1) / rows_per_wave;
        int wpb = e.block / 64;
        while (wpb > 1 && (waves + wpb - 1) / wpb < 1024) wpb /= 2;  // small jobs: more, smaller workgroups
        block = wpb * 64;
        a.nblocks = (waves + wpb - 1) / wpb;
    } else if (e.variant == SOFTMAX_VARIANT_ROW_PF) {
        block = e.block;
        const int64_t res = resident_workgroups(e, fn, block);
        a.nblocks = rows < res ? rows : res;
    } else {
        block = e.block;
        a.nblocks = rows;
    }
    const int64_t grid = a.nblocks < kMaxGrid ? a.nblocks : kMaxGrid;
    void* args[] = {&a};
    hipError_t rc = hipLaunchKernel(fn, dim3(unsigned(grid)), dim3(unsigned(block)), args, 0, stream);
    if (rc != hipSuccess) {
        (void)hipGetLastError();  // do not leave our failure for the caller's next check
        return SOFTMAX_ERR_HIP;
    }
    return SOFTMAX_OK;
}

bool splits_through_out(const void* in, const void* out, int64_t rows, int64_t cols, int64_t row_stride,
                        int dtype);
int launch_split(const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype, float* part,
                 hipStream_t stream);

int fwd(const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype, bool causal,
        float scale, int64_t diag, void* stream, int64_t period = 0) {
    bool empty;
    int st = validate(in, out, rows, cols, row_stride, dtype, &empty);
    if (st != SOFTMAX_OK) return st;
    float coef = float(kLog2eD);
    if (causal && !coef_of(scale, &coef)) return SOFTMAX_ERR_BAD_SCALE;
    if (empty) return SOFTMAX_OK;
    if (!causal && splits_through_out(in, out, rows, cols, row_stride, dtype))
        return launch_split(in, out, rows, cols, row_stride, dtype, nullptr, static_cast<hipStream_t>(stream));
    const Entry* e = select_entry(in, out, rows, cols, row_stride, dtype, causal);
    if (e == nullptr) return SOFTMAX_ERR_BAD_KERNEL;
    return launch(*e, in, out, rows, cols, row_stride, coef, diag, static_cast<hipStream_t>(stream), period);
}

int fwd_kernel(int kernel_id, const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride,
               int dtype, bool causal, float scale, int64_t diag, void* stream) {
    bool empty;
    int st = validate(in, out, rows, cols, row_stride, dtype, &empty);
    if (st != SOFTMAX_OK) return st;
    float coef = float(kLog2eD);
    if (causal && !coef_of(scale, &coef)) return SOFTMAX_ERR_BAD_SCALE;
    const Entry* e = entry_by_id(kernel_id);
    if (e == nullptr || e->causal != causal) return SOFTMAX_ERR_BAD_KERNEL;
    if (empty) return e->dtype == dtype ? SOFTMAX_OK : SOFTMAX_ERR_BAD_KERNEL;
    if (!fits(*e, in, out, cols, row_stride, dtype)) return SOFTMAX_ERR_BAD_KERNEL;
    return launch(*e, in, out, rows, cols, row_stride, coef, diag, static_cast<hipStream_t>(stream));
}

int select_id(const void* in, const void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
              bool causal, int* kernel_id) {
    if (kernel_id == nullptr) return SOFTMAX_ERR_NULL_POINTER;
    bool empty;
    int st = validate(in, out, rows, cols, row_stride, dtype, &empty);
    if (st != SOFTMAX_OK) return st;
    if (!causal && !empty && splits_through_out(in, out, rows, cols, row_stride, dtype)) {
        *kernel_id = SOFTMAX_KERNEL_SPLIT;
        return SOFTMAX_OK;
    }
    const Entry* e =
        select_entry(in, out, rows, cols > 0 ? cols : 1, row_stride > 0 ? row_stride : 1, dtype, causal);
    if (e == nullptr) return SOFTMAX_ERR_BAD_KERNEL;
    *kernel_id = id_of(e);
    return SOFTMAX_OK;
}

// ---- split-row path: tiles of one workgroup each, two kernels, a workspace

constexpr int kSplitW = 4;
constexpr int kSplitVecV = 4;     // 16-byte accesses per thread per tile
constexpr int kSplitScalarV = 8;  // elements per thread per tile (any alignment)
constexpr int64_t kSplitMaxRows = 1024;  // below this many rows, split when asked to choose

// Above this many tiles per row the workspace path merges each row's pairs
// once in a kernel of its own instead of in every workgroup of the norm
// kernel (tiles^2 pair reads per row).  Measured on one fp32 row: 2^24
// columns (4096 tiles) take 33 us with the merge in the norm kernel; with the
// merge kernel, 2^26 columns (16384 tiles) take 128 us instead of 242 and
// 2^28 columns (65536 tiles) 530 us instead of 2350.
constexpr int64_t kSplitMergeKernelTiles = 4096;

// Calls of up to this many tiles in all take softmax_fwd's own split in two
// kernels: every workgroup of the norm kernel merges its row's pairs from
// their slots (scattered 8-byte reads, one per tile of the row) and the last
// one of the row writes the tiles' first accesses, instead of a merge kernel
// in between.  That saves the merge kernel's launch and round trips, about
// 1 us (bf16 256 KiB x 8 rows: 10.7 -> 9.8 us); with more tiles the
// scattered reads, tiles^2 per row, cost more than that (bf16 512 KiB x 64
// rows, 2048 tiles: 21.4 us with the merge kernel, 22.9 without).
constexpr int64_t kSlotDirectTiles = 1024;

struct SplitPair {
    const void* stats;
    const void* norm;         // merges the row's pairs itself
    const void* merge;        // workspace pairs merged once per row ...
    const void* norm_merged;  // ... and read back by the norm kernel
    // 16-byte path only: stats, merge and norm with each tile's pair in its
    // own output slot (softmax_fwd's own split); for rows of few tiles the
    // norm kernel that merges the slots itself instead
    const void* stats_slot;
    const void* merge_slot;
    const void* norm_slot;
    const void* norm_slot_direct;
    int vec;
    int tile;  // accesses per tile
};

template <class E, int N, int V>
SplitPair split_kernels_of() {
    constexpr int W = kSplitW;
    SplitPair k = {(const void*)&rws::softmax_split_stats<E, N, W, V, false>,
                   (const void*)&rws::softmax_split_norm<E, N, W, V, false, false>,
                   (const void*)&rws::softmax_split_merge<E, N, W, V, false>,
                   (const void*)&rws::softmax_split_norm<E, N, W, V, false, true>,
                   nullptr, nullptr, nullptr, nullptr, N, W * 64 * V};
    if constexpr (N > 1) {
        k.stats_slot = (const void*)&rws::softmax_split_stats<E, N, W, V, true>;
        k.merge_slot = (const void*)&rws::softmax_split_merge<E, N, W, V, true>;
        k.norm_slot = (const void*)&rws::softmax_split_norm<E, N, W, V, true, true>;
        k.norm_slot_direct = (const void*)&rws::softmax_split_norm<E, N, W, V, true, false>;
    }
    return k;
}

template <class E>
SplitPair split_kernels(bool vec) {
    constexpr int kN = 16 / E::kBytes;
    return vec ? split_kernels_of<E, kN, kSplitVecV>() : split_kernels_of<E, 1, kSplitScalarV>();
}

SplitPair split_for(int dtype, bool vec) {
    switch (dtype) {
        case SOFTMAX_F32: return split_kernels<rws::F32>(vec);
        case SOFTMAX_F16: return split_kernels<rws::F16>(vec);
        default: return split_kernels<rws::BF16>(vec);
    }
}

// Tiles per row of the split path (the scalar path's tiles are the smallest,
// so the workspace is sized for them).
int64_t split_tiles(int64_t cols, const SplitPair& k) {
    const int64_t nacc = cols / k.vec;
    return (nacc + k.tile - 1) / k.tile;
}

// Workspace bytes of the split path (8 per tile, rounded up to 256), or -1
// when the count would not fit in int64.
int64_t split_workspace(int64_t rows, int64_t cols, int dtype) {
    const int64_t tiles = split_tiles(cols, split_for(dtype, false));
    if (tiles > 0 && rows > (INT64_MAX - 255) / 8 / tiles) return -1;
    return ((rows * tiles * 8 + 255) / 256) * 256;
}

// The split path's kernels in order.  With a workspace (`part`): stats, norm,
// with the per-row merge between them for rows of many tiles.  Without one
// (part == nullptr, the 16-byte path, out != in): the pairs kept in the
// output's tile slots, stats and norm for rows of few tiles, stats, merge and
// norm for the rest.
int launch_split(const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype, float* part,
                 hipStream_t stream) {
    const SplitPair k = split_for(dtype, aligned16(in, out, cols, row_stride, dtype));
    rws::SplitArgs a;
    a.in = in;
    a.out = out;
    a.part = part;
    a.rows = rows;
    a.stride = row_stride / k.vec;
    a.nacc = int(cols / k.vec);
    a.tiles = int(split_tiles(cols, k));
    a.work = rows * a.tiles;
    a.coef = float(kLog2eD);
    const int64_t grid = a.work < kMaxGrid ? a.work : kMaxGrid;
    const int64_t row_grid = rows < kMaxGrid ? rows : kMaxGrid;
    struct Step {
        const void* fn;
        int64_t grid;
    };
    const Step with_part[] = {{k.stats, grid}, {k.norm, grid}};
    const Step with_part_merged[] = {{k.stats, grid}, {k.merge, row_grid}, {k.norm_merged, grid}};
    const Step in_slots[] = {{k.stats_slot, grid}, {k.merge_slot, row_grid}, {k.norm_slot, grid}};
    const Step in_slots_direct[] = {{k.stats_slot, grid}, {k.norm_slot_direct, grid}};
    const bool merge_kernel = a.tiles > kSplitMergeKernelTiles;
    const bool direct = a.work <= kSlotDirectTiles;
    const Step* steps = part == nullptr ? (direct ? in_slots_direct : in_slots)
                                        : merge_kernel ? with_part_merged : with_part;
    const int nsteps = part != nullptr ? (merge_kernel ? 3 : 2) : (direct ? 2 : 3);
    if (part == nullptr && (k.stats_slot == nullptr || in == out)) return SOFTMAX_ERR_BAD_KERNEL;
    void* args[] = {&a};
    for (int i = 0; i < nsteps; ++i) {
        if (hipLaunchKernel(steps[i].fn, dim3(unsigned(steps[i].grid)), dim3(kSplitW * 64), args, 0, stream) !=
            hipSuccess) {
            (void)hipGetLastError();
            return SOFTMAX_ERR_HIP;
        }
    }
    return SOFTMAX_OK;
}

// softmax_fwd's own split, through the output's tile slots: out of place, on
// the 16-byte path, when a row has at least `min_row_bytes` and there are at
// most `max_rows` rows (first matching line, widest first).  One workgroup per
// row keeps at most `rows` compute units busy, and on such rows each runs at a
// rate set by its element count; the split reads every element twice and adds
// a launch of 2-4 us.  Measured for fp32, fp16 and bf16 at 8 .. 256 rows of
// 64 KiB .. 4 MiB against one workgroup per row; each line is where the split
// gained at least 5% (e.g. fp32 4 MiB rows: 9.7x at 8 rows, 1.5x at 128; bf16
// 512 KiB rows: 3.3x at 8, 1.2x at 128; bf16 224 KiB rows: 1.5x at 8).  fp32
// rows past 256 KiB (65536 columns) leave the register-resident kernels for
// the two-pass one, and there the split gains up to 64 rows (384 KiB x 32:
// 1.5x).
struct SlotSplitRule {
    int64_t min_row_bytes;
    int64_t max_rows;
};
constexpr SlotSplitRule kSlotSplitF32[] = {{int64_t(2) << 20, 192},
                                           {int64_t(1) << 20, 128},
                                           {(int64_t(256) << 10) + 16, 64},  // past the register-resident rows
                                           {int64_t(224) << 10, 32},
                                           {int64_t(192) << 10, 16}};
constexpr SlotSplitRule kSlotSplit16[] = {{int64_t(2) << 20, 256}, {int64_t(1) << 20, 192}, {int64_t(512) << 10, 128},
                                          {int64_t(192) << 10, 64},  {int64_t(128) << 10, 16}};

bool splits_through_out(const void* in, const void* out, int64_t rows, int64_t cols, int64_t row_stride,
                        int dtype) {
    if (in == out || !aligned16(in, out, cols, row_stride, dtype)) return false;
    const int64_t row_bytes = cols * elem_bytes(dtype);
    const bool f32 = dtype == SOFTMAX_F32;
    const SlotSplitRule* rules = f32 ? kSlotSplitF32 : kSlotSplit16;
    const int n = f32 ? int(sizeof(kSlotSplitF32) / sizeof(kSlotSplitF32[0]))
                      : int(sizeof(kSlotSplit16) / sizeof(kSlotSplit16[0]));
    for (int i = 0; i < n; ++i)
        if (row_bytes >= rules[i].min_row_bytes) return rows <= rules[i].max_rows;
    return false;
}

// ---- the split path without a caller workspace
//
// `scratch` is the split path's workspace for softmax_fwd_split_noalloc: one
// copy per device, held until the process ends.  In host code its name is a
// host-side stand-in, not a device address; the device address comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept in g_scratch.  Launches take that address, never the name.
static __device__ __align__(256) unsigned char scratch[SOFTMAX_NOALLOC_SCRATCH_BYTES];

std::atomic<uintptr_t> g_scratch[kMaxDevices];  // 0 = not yet looked up

// The current device's address of `scratch`, or nullptr if HIP cannot give it.
void* scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    const uintptr_t known = g_scratch[dev].load(std::memory_order_acquire);
    if (known != 0) return reinterpret_cast<void*>(known);
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
        (void)hipGetLastError();
        return nullptr;
    }
    g_scratch[dev].store(reinterpret_cast<uintptr_t>(ptr), std::memory_order_release);
    return ptr;
}

// Whether a softmax_fwd_split call takes the split path (force 1, or few rows
// that span two or more tiles).
bool takes_split(const void* in, const void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
                 int force) {
    const SplitPair k = split_for(dtype, aligned16(in, out, cols, row_stride, dtype));
    return force == 1 || (rows < kSplitMaxRows && split_tiles(cols, k) >= 2);
}

}  // namespace

extern "C" {

int64_t softmax_split_workspace_bytes(int64_t rows, int64_t cols, int dtype) {
    if (rows < 0 || cols < 0 || cols > kMaxCols) return -1;
    if (dtype != SOFTMAX_F32 && dtype != SOFTMAX_F16 && dtype != SOFTMAX_BF16) return -1;
    if (rows > INT64_MAX / 8 / (cols / 2048 + 2)) return -1;
    return split_workspace(rows, cols, dtype);
}

int softmax_fwd_split(const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
                      void* workspace, int64_t workspace_size, int force, void* stream) {
    bool empty;
    int st = validate(in, out, rows, cols, row_stride, dtype, &empty);
    if (st != SOFTMAX_OK || empty) return st;
    if (force != 0 && force != 1) return SOFTMAX_ERR_BAD_KERNEL;
    if (!takes_split(in, out, rows, cols, row_stride, dtype, force))
        return fwd(in, out, rows, cols, row_stride, dtype, false, 1.0f, 0, stream);
    if (workspace == nullptr) return SOFTMAX_ERR_NULL_POINTER;
    const int64_t need = split_workspace(rows, cols, dtype);
    if (need < 0 || uintptr_t(workspace) % 256 || workspace_size < need) return SOFTMAX_ERR_BAD_SHAPE;
    const int64_t esz = elem_bytes(dtype);
    const int64_t extent = ((rows - 1) * row_stride + cols) * esz;
    const uintptr_t a = uintptr_t(in), b = uintptr_t(out), w = uintptr_t(workspace);
    if ((w < a + uint64_t(extent) && a < w + uint64_t(need)) || (w < b + uint64_t(extent) && b < w + uint64_t(need)))
        return SOFTMAX_ERR_OVERLAP;
    return launch_split(in, out, rows, cols, row_stride, dtype, static_cast<float*>(workspace),
                        static_cast<hipStream_t>(stream));
}

int softmax_fwd_split_noalloc(const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
                              int force, void* stream) {
    bool empty;
    int st = validate(in, out, rows, cols, row_stride, dtype, &empty);
    if (st != SOFTMAX_OK || empty) return st;
    if (force != 0 && force != 1) return SOFTMAX_ERR_BAD_KERNEL;
    if (!takes_split(in, out, rows, cols, row_stride, dtype, force))
        return fwd(in, out, rows, cols, row_stride, dtype, false, 1.0f, 0, stream);
    const int64_t need = split_workspace(rows, cols, dtype);
    if (need < 0 || need > int64_t(SOFTMAX_NOALLOC_SCRATCH_BYTES)) return SOFTMAX_ERR_SCRATCH_LIMIT;
    void* part = scratch_on_current_device();
    if (part == nullptr) return SOFTMAX_ERR_HIP;
    return launch_split(in, out, rows, cols, row_stride, dtype, static_cast<float*>(part),
                        static_cast<hipStream_t>(stream));
}

int softmax_fwd(const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
                void* stream) {
    return fwd(in, out, rows, cols, row_stride, dtype, false, 1.0f, 0, stream);
}

int softmax_fwd_causal(const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride, float scale,
                       int64_t diag, int dtype, void* stream) {
    return fwd(in, out, rows, cols, row_stride, dtype, true, scale, diag, stream);
}

int softmax_fwd_causal_batched(const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride,
                               int64_t rows_per_matrix, float scale, int64_t diag, int dtype, void* stream) {
    bool empty;
    int st = validate(in, out, rows, cols, row_stride, dtype, &empty);
    if (st != SOFTMAX_OK) return st;
    if (!empty && (rows_per_matrix < 1 || rows % rows_per_matrix != 0)) return SOFTMAX_ERR_BAD_SHAPE;
    return fwd(in, out, rows, cols, row_stride, dtype, true, scale, diag, stream, rows_per_matrix);
}

int softmax_fwd_kernel(int kernel_id, const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride,
                       int dtype, void* stream) {
    return fwd_kernel(kernel_id, in, out, rows, cols, row_stride, dtype, false, 1.0f, 0, stream);
}

int softmax_fwd_causal_kernel(int kernel_id, const void* in, void* out, int64_t rows, int64_t cols,
                              int64_t row_stride, float scale, int64_t diag, int dtype, void* stream) {
    return fwd_kernel(kernel_id, in, out, rows, cols, row_stride, dtype, true, scale, diag, stream);
}

int softmax_fwd_variant(const void* in, void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
                        int variant, int block, void* stream) {
    bool empty;
    int st = validate(in, out, rows, cols, row_stride, dtype, &empty);
    if (st != SOFTMAX_OK) return st;
    if (variant < SOFTMAX_VARIANT_PACKED || variant > SOFTMAX_VARIANT_ROW16) return SOFTMAX_ERR_BAD_KERNEL;
    if (empty) return SOFTMAX_OK;
    const Entry* e = entry_for_variant(in, out, cols, row_stride, dtype, variant, block);
    if (e == nullptr) return SOFTMAX_ERR_BAD_KERNEL;
    return launch(*e, in, out, rows, cols, row_stride, float(kLog2eD), 0, static_cast<hipStream_t>(stream));
}

int softmax_select_variant(int64_t cols, int dtype, int* variant, int* block) {
    if (variant == nullptr || block == nullptr) return SOFTMAX_ERR_NULL_POINTER;
    if (dtype != SOFTMAX_F32 && dtype != SOFTMAX_F16 && dtype != SOFTMAX_BF16) return SOFTMAX_ERR_BAD_DTYPE;
    if (cols < 1 || cols > kMaxCols) return SOFTMAX_ERR_BAD_SHAPE;
    // A contiguous tensor on 256-byte-aligned buffers with many rows (never
    // dereferenced): the pick of softmax_fwd for this width and dtype.
    const void* in = reinterpret_cast<const void*>(uintptr_t(1) << 40);
    const void* out = reinterpret_cast<const void*>(uintptr_t(1) << 41);
    const Entry* e = select_entry(in, out, int64_t(1) << 20, cols, cols, dtype, false);
    if (e == nullptr) return SOFTMAX_ERR_BAD_KERNEL;
    *variant = e->variant;
    *block = e->variant == SOFTMAX_VARIANT_PACKED ? e->lanes : e->block;
    return SOFTMAX_OK;
}

int softmax_select(const void* in, const void* out, int64_t rows, int64_t cols, int64_t row_stride, int dtype,
                   int* kernel_id) {
    return select_id(in, out, rows, cols, row_stride, dtype, false, kernel_id);
}

int softmax_select_causal(const void* in, const void* out, int64_t rows, int64_t cols, int64_t row_stride,
                          int dtype, int* kernel_id) {
    return select_id(in, out, rows, cols, row_stride, dtype, true, kernel_id);
}

int softmax_num_kernels(void) { return total_kernels(); }

int softmax_kernel_info(int kernel_id, int* dtype, int* variant, int* causal, int* vec_elems, int* lanes,
                        int* vecs_per_lane, int* groups, int* block, int64_t* max_cols) {
    const Entry* e = entry_by_id(kernel_id);
    if (e == nullptr) return SOFTMAX_ERR_BAD_KERNEL;
    if (dtype) *dtype = e->dtype;
    if (variant) *variant = e->variant;
    if (causal) *causal = e->causal ? 1 : 0;
    if (vec_elems) *vec_elems = e->vec;
    if (lanes) *lanes = e->lanes;
    if (vecs_per_lane) *vecs_per_lane = e->vpl;
    if (groups) *groups = e->groups;
    if (block) *block = e->block;
    if (max_cols) *max_cols = max_cols_of(*e);
    return SOFTMAX_OK;
}

const char* softmax_kernel_name(int kernel_id) {
    const Entry* e = entry_by_id(kernel_id);
    return e ? e->name : nullptr;
}

int softmax_kernel_fits(int kernel_id, const void* in, const void* out, int64_t cols, int64_t row_stride,
                        int dtype) {
    const Entry* e = entry_by_id(kernel_id);
    if (e == nullptr || cols < 0 || row_stride < cols || cols > kMaxCols) return 0;
    return fits(*e, in, out, cols, row_stride, dtype) ? 1 : 0;
}

const char* softmax_status_string(int status) {
    switch (status) {
        case SOFTMAX_OK: return "ok";
        case SOFTMAX_ERR_NULL_POINTER: return "null pointer";
        case SOFTMAX_ERR_BAD_SHAPE: return "bad shape (negative dims, row_stride < cols, cols > 2^30 or extent overflow)";
        case SOFTMAX_ERR_BAD_DTYPE: return "bad dtype (expected 0 = fp32, 1 = fp16, 2 = bf16)";
        case SOFTMAX_ERR_OVERLAP: return "input and output overlap without being equal";
        case SOFTMAX_ERR_BAD_KERNEL: return "kernel id unknown, of the other kind (plain or causal), or unable to take this dtype, width, stride or alignment";
        case SOFTMAX_ERR_HIP: return "HIP runtime refused the launch";
        case SOFTMAX_ERR_BAD_SCALE: return "bad scale (must be > 0 with scale * log2(e) below 3e38)";
        case SOFTMAX_ERR_SCRATCH_LIMIT: return "the split path needs more workspace than the static scratch buffer holds (SOFTMAX_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown status";
    }
}

const char* softmax_version(void) { return "row_wise_softmax_amd 0.2.0 (gfx950)"; }

int softmax_bench_stream(const void* src, void* dst, int64_t bytes, int mode, void* stream) {
    if (mode == 0) return softmax_bench_copy(src, dst, bytes, stream);
    if (mode != 1 && mode != 2) return SOFTMAX_ERR_BAD_KERNEL;
    if (bytes < 0 || bytes % 16) return SOFTMAX_ERR_BAD_SHAPE;
    if (bytes == 0) return SOFTMAX_OK;
    if (dst == nullptr || (mode == 1 && src == nullptr)) return SOFTMAX_ERR_NULL_POINTER;
    if ((mode == 1 && uintptr_t(src) % 16) || uintptr_t(dst) % 16) return SOFTMAX_ERR_BAD_SHAPE;
    constexpr int kU = 4;
    const int64_t n = bytes / 16;
    int64_t grid = (n + 256 * kU - 1) / (256 * kU);
    if (grid > kMaxGrid) grid = kMaxGrid;
    int64_t nn = n;
    hipError_t rc;
    if (mode == 1) {
        const rws::u32x4* s = static_cast<const rws::u32x4*>(src);
        unsigned* sink = static_cast<unsigned*>(dst);
        // Any value: should the data's XOR ever equal it, the one word the
        // kernel then stores lands in dst's first 4 bytes, which the caller
        // provides for that.
        unsigned never = 0x7fbadbadu;
        void* args[] = {&s, &sink, &nn, &never};
        rc = hipLaunchKernel((const void*)&rws::read16<kU>, dim3(unsigned(grid)), dim3(256), args, 0,
                             static_cast<hipStream_t>(stream));
    } else {
        rws::u32x4* d = static_cast<rws::u32x4*>(dst);
        unsigned value = 0x3c003c00u;
        void* args[] = {&d, &nn, &value};
        rc = hipLaunchKernel((const void*)&rws::write16<kU>, dim3(unsigned(grid)), dim3(256), args, 0,
                             static_cast<hipStream_t>(stream));
    }
    if (rc != hipSuccess) {
        (void)hipGetLastError();
        return SOFTMAX_ERR_HIP;
    }
    return SOFTMAX_OK;
}

int softmax_bench_chunk_copy(const void* src, void* dst, int64_t bytes, int waves, int accesses, void* stream) {
    struct Shape { int w, v; const void* fn; };
    static const Shape kShapes[] = {
        {4, 2, (const void*)&rws::chunk_copy16<4, 2>},   {8, 2, (const void*)&rws::chunk_copy16<8, 2>},
        {4, 4, (const void*)&rws::chunk_copy16<4, 4>},   {16, 2, (const void*)&rws::chunk_copy16<16, 2>},
        {4, 8, (const void*)&rws::chunk_copy16<4, 8>},   {8, 4, (const void*)&rws::chunk_copy16<8, 4>},
        {4, 16, (const void*)&rws::chunk_copy16<4, 16>}, {8, 8, (const void*)&rws::chunk_copy16<8, 8>},
        {16, 4, (const void*)&rws::chunk_copy16<16, 4>},
    };
    const Shape* k = nullptr;
    for (const Shape& sh : kShapes)
        if (sh.w == waves && sh.v == accesses) k = &sh;
    if (k == nullptr) return SOFTMAX_ERR_BAD_KERNEL;
    const int64_t chunk = int64_t(waves) * 64 * accesses * 16;
    if (bytes < 0 || bytes % chunk) return SOFTMAX_ERR_BAD_SHAPE;
    if (bytes == 0) return SOFTMAX_OK;
    if (src == nullptr || dst == nullptr) return SOFTMAX_ERR_NULL_POINTER;
    if (uintptr_t(src) % 16 || uintptr_t(dst) % 16) return SOFTMAX_ERR_BAD_SHAPE;
    const uintptr_t a = uintptr_t(src), b = uintptr_t(dst);
    if (a < b + uint64_t(bytes) && b < a + uint64_t(bytes)) return SOFTMAX_ERR_OVERLAP;
    int64_t n = bytes / chunk;
    const int64_t grid = n < kMaxGrid ? n : kMaxGrid;
    const rws::u32x4* s = static_cast<const rws::u32x4*>(src);
    rws::u32x4* d = static_cast<rws::u32x4*>(dst);
    void* args[] = {&s, &d, &n};
    if (hipLaunchKernel(k->fn, dim3(unsigned(grid)), dim3(unsigned(waves * 64)), args, 0,
                        static_cast<hipStream_t>(stream)) != hipSuccess) {
        (void)hipGetLastError();
        return SOFTMAX_ERR_HIP;
    }
    return SOFTMAX_OK;
}

int softmax_bench_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16) return SOFTMAX_ERR_BAD_SHAPE;
    if (bytes == 0) return SOFTMAX_OK;
    if (src == nullptr || dst == nullptr) return SOFTMAX_ERR_NULL_POINTER;
    if (uintptr_t(src) % 16 || uintptr_t(dst) % 16) return SOFTMAX_ERR_BAD_SHAPE;
    const uintptr_t a = uintptr_t(src), b = uintptr_t(dst);
    if (a < b + uint64_t(bytes) && b < a + uint64_t(bytes)) return SOFTMAX_ERR_OVERLAP;
    constexpr int kU = 4;
    const int64_t n = bytes / 16;
    int64_t grid = (n + 256 * kU - 1) / (256 * kU);
    if (grid > kMaxGrid) grid = kMaxGrid;
    const rws::u32x4* s = static_cast<const rws::u32x4*>(src);
    rws::u32x4* d = static_cast<rws::u32x4*>(dst);
    int64_t nn = n;
    void* args[] = {&s, &d, &nn};
    hipError_t rc = hipLaunchKernel((const void*)&rws::copy16<kU>, dim3(unsigned(grid)), dim3(256), args, 0,
                                    static_cast<hipStream_t>(stream));
    if (rc != hipSuccess) {
        (void)hipGetLastError();
        return SOFTMAX_ERR_HIP;
    }
    return SOFTMAX_OK;
}

}  // extern "C"
