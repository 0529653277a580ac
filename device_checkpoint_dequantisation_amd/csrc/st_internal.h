// Internal definitions shared by the host planner and the device kernel of libstmat.
#pragma once

#include <stdint.h>

#include "stmat.h"

static_assert(sizeof(st_desc) == 64, "st_desc must stay 64 bytes");

// Records a printf-style message for st_last_error() on this thread and returns `code`.
st_status st_fail(st_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Work-unit geometry, in elements per unit.  kWords = 16-byte output words per lane per unit
// counted for a 2-byte output type (8 elements each); output word o*64 + lane of a unit belongs to
// lane `lane`, so each store instruction of the wavefront covers 1 KB of contiguous output (fp32
// outputs: twice the words, 4 elements each):
//   bf16/fp16 sources : 2 words -> 1024 elements (2 KB in, 2 KB out)
//   fp32 sources      : 1 word  ->  512 elements (2 KB in, 1 KB out)
//   fp8 (all scalings): 2 words -> 1024 elements (1 KB in, 2 KB out)
//   nvfp4 / mxfp4     : 4 words -> 2048 elements (1 KB + 64-128 B in, 4 KB out); into fp32
//                       outputs 2 words -> 1024 elements (512 B + 32-64 B in, 4 KB out)
// so every unit reads about 0.5-2 KB and writes 1-4 KB: one short, fully coalesced burst per
// wave.  (Packed fp4 into fp32 with 2048-element units, 8 KB written per wave, ran 10-14% slower
// on MI355X than with 1024.)
namespace stk {
constexpr uint32_t kWave = 64;
constexpr uint32_t kWordElems = 8;
#ifndef STK_WORDS_PASS
#define STK_WORDS_PASS 2
#endif
#ifndef STK_WORDS_F32
#define STK_WORDS_F32 1
#endif
#ifndef STK_WORDS_FP8
#define STK_WORDS_FP8 2
#endif
#ifndef STK_WORDS_FP4
#define STK_WORDS_FP4 4
#endif
#ifndef STK_WORDS_FP4_F32
#define STK_WORDS_FP4_F32 2
#endif
constexpr uint32_t kWordsPass = STK_WORDS_PASS, kWordsF32 = STK_WORDS_F32, kWordsFp8 = STK_WORDS_FP8,
                   kWordsFp4 = STK_WORDS_FP4, kWordsFp4F32 = STK_WORDS_FP4_F32;

constexpr uint32_t ilog2(uint32_t x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

constexpr uint32_t words_per_lane(uint32_t kind, uint32_t out_dtype) {
    return kind == ST_KIND_PASS_BF16 || kind == ST_KIND_CAST_F16 ? kWordsPass
         : kind == ST_KIND_CAST_F32                              ? kWordsF32
         : kind == ST_KIND_NVFP4 || kind == ST_KIND_MXFP4        ? (out_dtype == ST_OUT_F32 ? kWordsFp4F32 : kWordsFp4)
                                                                 : kWordsFp8;
}
// The kernel's chunk geometry per kind: output elements per chunk (8 for every kind: one 16-byte
// word of a 2-byte output type), and the load word size that a source must be aligned to for the
// fast path (a chunk's source bytes, at most 16).  A column slice keeps the fast path when its
// width is a whole number of chunks and its row length in bytes is a whole number of load words.
constexpr uint32_t chunk_elems(uint32_t) { return 8; }
constexpr uint32_t load_word_bytes(uint32_t kind) {
    return kind == ST_KIND_NVFP4 || kind == ST_KIND_MXFP4 ? 4
         : kind == ST_KIND_FP8_TENSOR || kind == ST_KIND_FP8_BLOCK128 || kind == ST_KIND_MXFP8 ? 8
                                                                                               : 16;
}
// Kinds whose complete column-shard sets are planned as split descriptors (the source rows read
// whole, each chunk stored to its shard): the packed fp4 kinds.  On 8-way shards of the large
// checkpoints this beat one descriptor per shard by 14% (NVFP4) and 10% (MXFP4), measured on MI355X
// with the column-slice path's non-temporal loads; with those loads one descriptor per shard is the
// faster plan for the 8-bit kinds (MXFP8 +12%, scaled FP8 +3% over split descriptors), for bf16 (4%),
// and block FP8, whose scale grid needs the shard's own columns.
constexpr bool split_kind(uint32_t kind) { return kind == ST_KIND_NVFP4 || kind == ST_KIND_MXFP4; }
// Source bits per element.
constexpr uint32_t source_bits(uint32_t kind) {
    return kind == ST_KIND_CAST_F32 ? 32
         : kind == ST_KIND_PASS_BF16 || kind == ST_KIND_CAST_F16 ? 16
         : kind == ST_KIND_NVFP4 || kind == ST_KIND_MXFP4 ? 4
                                                           : 8;
}

// Where the descriptors start in a work table of `groups` map entries.
constexpr uint64_t table_desc_offset(uint64_t groups) { return 64 + (groups * 4 + 63) / 64 * 64; }

// log2 of the default unit size (elements) of a kind decoded into an output type
constexpr uint32_t step_shift(uint32_t kind, uint32_t out_dtype) {
    return ilog2(kWave * kWordElems * words_per_lane(kind, out_dtype));
}

// Exact unsigned 32-bit division by an invariant divisor d >= 1 (Granlund & Montgomery,
// "Division by Invariant Integers using Multiplication", 1994, the round-up method with an
// N+1-bit multiplier): with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
//   t = mulhi(m, n),  q = (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0)
// equals floor(n / d) for every 32-bit n.  constexpr so the same code runs on host and device.
constexpr uint32_t div_magic(uint32_t d) {
    uint32_t l = 0;
    while (l < 32 && (uint64_t(1) << l) < d) ++l;
    return uint32_t((((uint64_t(1) << l) - d) << 32) / d + 1);
}
constexpr uint32_t div_shift(uint32_t d) {
    uint32_t l = 0;
    while (l < 32 && (uint64_t(1) << l) < d) ++l;
    return l;
}
constexpr uint32_t div_apply(uint32_t n, uint32_t magic, uint32_t l) {
    const uint32_t t = uint32_t((uint64_t(magic) * n) >> 32);
    return l == 0 ? n : (t + ((n - t) >> 1)) >> (l - 1);
}
}  // namespace stk
