// Internal definitions shared by the host planner and the device kernel of libstmat.
#pragma once

#include <stdint.h>

#include "stmat.h"

static_assert(sizeof(st_desc) == 64, "st_desc must stay 64 bytes");

// Records a printf-style message for st_last_error() on this thread and returns `code`.
st_status st_fail(st_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Elements one lane handles per chunk, and chunks per lane in one wave step.  A wave step is
// the smallest work unit; its size is chosen so every unit moves roughly 10-16 KB of HBM traffic
// whatever its kind, which keeps the static, interleaved unit schedule balanced.
//   bf16/fp16 : 8 elements = 16 B in, 16 B out per chunk, 8 chunks -> 4096 elements (16 KB)
//   fp32      : 8 elements = 32 B in, 16 B out per chunk, 4 chunks -> 2048 elements (12 KB)
//   fp8       : 16 elements = 16 B in, 32 B out per chunk, 4 chunks -> 4096 elements (12 KB)
//   nvfp4     : 32 elements = 16 B + 2 B in, 64 B out per chunk, 2 chunks -> 4096 (10.25 KB)
namespace stk {
constexpr uint32_t kWave = 64;
constexpr uint32_t kChunkPass = 8, kStepsPass = 8;
constexpr uint32_t kChunkF32 = 8, kStepsF32 = 4;
constexpr uint32_t kChunkFp8 = 16, kStepsFp8 = 4;
constexpr uint32_t kChunkFp4 = 32, kStepsFp4 = 2;

constexpr uint32_t ilog2(uint32_t x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

constexpr uint32_t step_shift(uint32_t kind) {
    return kind == ST_KIND_PASS_BF16 || kind == ST_KIND_CAST_F16 ? ilog2(kWave * kChunkPass * kStepsPass)
         : kind == ST_KIND_CAST_F32                              ? ilog2(kWave * kChunkF32 * kStepsF32)
         : kind == ST_KIND_NVFP4                                 ? ilog2(kWave * kChunkFp4 * kStepsFp4)
                                                                 : ilog2(kWave * kChunkFp8 * kStepsFp8);
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
