// The grouped materialise kernel: one launch turns every descriptor's bytes in the device blob
// into bf16 outputs.
//
// What it computes is fixed by the checkpoint formats the pages name ("Resident Modal LLM
// Architecture", "Current Backend Boundary": Qwen block-FP8, ModelOpt NVFP4; "Disk tier
// safetensors streaming design audit", "Mandatory research audit": ComfyUI scaled FP8) read as
// OCP E4M3 / OCP-MX E2M1 codes, one IEEE binary32 round-to-nearest-even multiply per scale and a
// round-to-nearest-even narrowing to bfloat16 (NaN -> 0x7FC0, no subnormal flushing).
//
// Shape of the work.  This is a memory-bound elementwise codec (2.6-6 bytes of HBM traffic per
// element, a handful of VALU operations per element), so there is no matrix-core work; what
// matters on gfx950 is how the HBM traffic is issued:
//  * One wavefront per work unit, one-shot.  A unit is 512-2048 elements of one output (about
//    1-2 KB read, 1-4 KB written).  Each wavefront loads its unit, decodes, stores and exits.
//    Measured on MI355X, one-shot wavefronts sustain ~20% more read+write bandwidth than any
//    persistent loop tried (grid-stride, contiguous ranges, software-pipelined), because a
//    persistent wavefront's next loads wait behind its own outstanding stores (vmcnt counts both).
//  * Lane-contiguous stores.  Lane l writes 16-byte output words o*64 + l, so every store
//    instruction of a wavefront covers 1 KB of contiguous output; lanes read whatever input bytes
//    their output words need (4, 8, 16 or 32 bytes).
//  * XCD-contiguous order.  The hardware hands workgroup b to XCD b mod 8; workgroups are
//    renumbered so each XCD streams through one contiguous eighth of the work.
//  * Tiny tensors.  Units are numbered consecutively across outputs and a workgroup's four
//    wavefronts take four consecutive units, whatever output they belong to, so small tensors are
//    packed at wavefront granularity.  A per-workgroup map gives the descriptor of the group's
//    first unit; a wavefront walks forward at most three descriptors.
//  * Unaligned sources.  A tensor may start at any byte.  A unit whose source is 16-byte aligned
//    loads whole 16-byte words (4-byte words for NVFP4).  Otherwise each lane loads from the
//    4-byte boundary at or below its bytes (16-byte words at 4-byte alignment plus one trailing
//    dword), and the byte offset sh (the same for every lane of a unit) is removed in registers
//    with v_alignbyte.  Measured on MI355X, this beats loading the two enclosing aligned 16-byte
//    words and selecting among them.
//  * Short dependency chain.  Ahead of a wavefront's data loads sit only the table header check,
//    its map entry and its descriptor; the output pointer and the scalar scale are loaded once the
//    data loads are in flight (a wait for one scalar load waits for all of them).
//  * Decoding uses gfx950's conversion instructions (fp8 and fp4 to fp32, fp32 to bf16), each
//    checked exhaustively against the exact decoding on the device; one fp32 multiply per scale.
//  * Tails, NaN inputs, non-finite scales, block-FP8 widths not a multiple of 16 and misaligned
//    outputs go through an exact per-element path written from the definitions alone.
#include <hip/hip_runtime.h>

#include <cstddef>

#include "st_internal.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

// Wave-uniform reads of data the kernel never writes (work table, output pointers, scalar
// scales) go through the constant address space, so they become scalar loads.
template <class T>
__device__ __forceinline__ T ld_uniform(const void* p) {
    return *reinterpret_cast<const __attribute__((address_space(4))) T*>(reinterpret_cast<uintptr_t>(p));
}

constexpr uint32_t kBlock = 256;  // threads per workgroup: ST_UNITS_PER_GROUP wavefronts
static_assert(kBlock == ST_UNITS_PER_GROUP * stk::kWave, "one wavefront per unit");
constexpr uint32_t kMaxGridX = 1u << 22;  // keeps gridDim.x * 256 below 2^32

// ------------------------------------------------------------------------- small helpers

__device__ __forceinline__ uint32_t ld_u8(const uint8_t* p) { return *p; }
__device__ __forceinline__ uint32_t ld_u16_any(const uint8_t* p) { return uint32_t(p[0]) | uint32_t(p[1]) << 8; }
__device__ __forceinline__ uint32_t ld_u32_any(const uint8_t* p) {
    return uint32_t(p[0]) | uint32_t(p[1]) << 8 | uint32_t(p[2]) << 16 | uint32_t(p[3]) << 24;
}
// fp32 at p, where `aligned` says whether p is 4-byte aligned (uniform per descriptor)
__device__ __forceinline__ float ld_f32(const uint8_t* p, bool aligned) {
    return aligned ? *reinterpret_cast<const float*>(p) : __builtin_bit_cast(float, ld_u32_any(p));
}
__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
// A wave-uniform fp32 at any byte address: the two aligned dwords around it (the blob is padded
// past its data), one scalar load, then a funnel shift.
__device__ __forceinline__ float ld_scalar_f32(const uint8_t* p) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const u32x2 w = ld_uniform<u32x2>(reinterpret_cast<const void*>(a & ~uintptr_t(3)));
    return __builtin_bit_cast(float, uint32_t((uint64_t(w.y) << 32 | w.x) >> (8 * (a & 3u))));
}

__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// Upper 16 bits = bf16 of f rounded to nearest, ties to even (f not NaN).
__device__ __forceinline__ uint32_t rne_hi(float f) {
    const uint32_t u = as_u32(f);
    return u + 0x7FFFu + ((u >> 16) & 1u);
}
__device__ __forceinline__ uint32_t bf16_canon(float f) { return f != f ? 0x7FC0u : rne_hi(f) >> 16; }

__device__ __forceinline__ float h2f(uint32_t h16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h16)));
}
// Exact path decoding.  e4m3 code -> its value times 2^-8, exactly: the code's exponent and
// mantissa fields are moved into an fp16's (subnormal codes land on fp16 subnormals).
__device__ __forceinline__ float e4m3_x2m8(uint32_t c) { return h2f(((c & 0x7Fu) << 7) | ((c & 0x80u) << 8)); }
// e2m1 code -> its value times 2^-14, exactly (same construction with a 2-bit exponent).
__device__ __forceinline__ float e2m1_x2m14(uint32_t n) { return h2f(((n & 7u) << 9) | ((n & 8u) << 12)); }
__device__ __forceinline__ float e4m3_exact(uint32_t c) {
    return (c & 0x7Fu) == 0x7Fu ? __builtin_nanf("") : e4m3_x2m8(c) * 256.0f;
}
__device__ __forceinline__ float e2m1_exact(uint32_t n) { return e2m1_x2m14(n) * 16384.0f; }

// True if any byte of x is an e4m3 NaN code (0x7F or 0xFF).
__device__ __forceinline__ bool has_nan_code(uint32_t x) {
    return (((x & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u) != 0;
}

// gfx950 conversion instructions used on the fast path.  Each was checked exhaustively on the
// device against the exact decoding above: v_cvt_pk_f32_fp8 on every pair of e4m3 codes (it
// decodes OCP e4m3fn), v_cvt_scalef32_pk_f32_fp4 with scale 1.0 on every byte, and
// v_cvt_pk_bf16_f32 on all 2^32 fp32 patterns (round to nearest even, subnormals kept; it keeps
// NaN payloads, so the fast path never hands it a NaN).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {  // a at the lower address
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// e4m3 codes in bytes 0,1 (HI: 2,3) of x -> exact fp32 values
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2(uint32_t x) { return __builtin_amdgcn_cvt_pk_f32_fp8(x, HI); }
// e2m1 codes in byte P of x (low nibble first) -> exact fp32 values
template <int P>
__device__ __forceinline__ f32x2 fp4x2(uint32_t x) { return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, P); }
__device__ __forceinline__ bool finite(float s) { return __builtin_fabsf(s) <= 3.4028234663852886e38f; }

// ------------------------------------------------------------------------- descriptors

struct Desc {
    uint64_t src, scale, scale2;
    uint32_t pitch, flags;
    uint32_t unit_begin, unit_end, tail, out, cols, grid_cols, div_magic, kind, unit_shift, div_shift;
};

// The 64-byte descriptor in one scalar load.
__device__ __forceinline__ Desc load_desc(const st_desc* d) {
    const u32x16 w = ld_uniform<u32x16>(d);
    Desc r;
    r.src = uint64_t(w[1]) << 32 | w[0];
    r.scale = uint64_t(w[3]) << 32 | w[2];
    r.scale2 = uint64_t(w[5]) << 32 | w[4];
    r.pitch = w[6];
    r.flags = w[7];
    r.unit_begin = w[8];
    r.unit_end = w[9];
    r.tail = w[10];
    r.out = w[11];
    r.cols = w[12];
    r.grid_cols = w[13];
    r.div_magic = w[14];
    r.kind = w[15] & 0xFFu;
    r.unit_shift = (w[15] >> 8) & 0xFFu;
    r.div_shift = (w[15] >> 16) & 0xFFu;
    return r;
}
static_assert(offsetof(st_desc, meta) == 15 * 4, "descriptor layout");

// Source element of output element e: e itself, or for a column slice (pitch != 0) the element
// row * pitch + col of the slice's source rows, with row = e / cols and col = e % cols.
__device__ __forceinline__ uint64_t src_elem(const Desc& D, uint64_t e) {
    if (D.pitch == 0) return e;
    const uint32_t row = stk::div_apply(uint32_t(e), D.div_magic, D.div_shift);
    return e + uint64_t(row) * (D.pitch - D.cols);
}

// bf16 bits of element e of descriptor D, straight from the definition, byte by byte.
__device__ __forceinline__ uint32_t elem_exact(const uint8_t* __restrict__ blob, const Desc& D, uint64_t e) {
    const uint8_t* s = blob + D.src;
    const uint64_t x = src_elem(D, e);
    switch (D.kind) {
        case ST_KIND_PASS_BF16: return ld_u16_any(s + 2 * x);
        case ST_KIND_CAST_F16: return bf16_canon(h2f(ld_u16_any(s + 2 * x)));
        case ST_KIND_CAST_F32: return bf16_canon(as_f32(ld_u32_any(s + 4 * x)));
        case ST_KIND_FP8_TENSOR: return bf16_canon(e4m3_exact(ld_u8(s + x)) * as_f32(ld_u32_any(blob + D.scale)));
        case ST_KIND_FP8_BLOCK128: {  // the scale grid position comes from the output's row and column
            const uint32_t e32 = uint32_t(e);
            const uint32_t row = stk::div_apply(e32, D.div_magic, D.div_shift);
            const uint32_t col = e32 - row * D.cols;
            const float S = as_f32(ld_u32_any(blob + D.scale + 4ull * ((row >> 7) * D.grid_cols + (col >> 7))));
            return bf16_canon(e4m3_exact(ld_u8(s + x)) * S);
        }
        default: {  // NVFP4: K % 16 == 0, so block scale (i, j / 16) sits at flat source index x / 16
            const uint32_t nib = (ld_u8(s + (x >> 1)) >> ((x & 1) * 4)) & 15u;
            const float bs = e4m3_exact(ld_u8(blob + D.scale + (x >> 4)));
            const float g = as_f32(ld_u32_any(blob + D.scale2));
            const float t = e2m1_exact(nib) * bs;
            return bf16_canon(t * g);
        }
    }
}

// ------------------------------------------------------------------------- per-kind chunks
//
// A Kind decodes one chunk of CE elements (CE/8 16-byte output words, stored adjacently) from IB
// input bytes, fetched as naturally aligned LG-byte words.  `fast` returns false when the chunk
// must take the exact path.  CH = chunks per lane per step; chunk c of a step belongs to lane
// c % 64.

// Per-unit context.  `s` and `vec` are filled in by finish_ctx, after the data loads are issued;
// whether the scale folds into the fast path is decided in the decode.
struct Ctx {
    const uint8_t* blob;
    Desc D;
    uint16_t* const* outs;  // output pointers, indexed by the descriptor's `out`
    float s;         // FP8_TENSOR: the per-tensor scale; NVFP4: the global scale
    bool scale_al;   // the descriptor's scale data is 4-byte aligned
    bool vec;        // the output is 16-byte aligned (vector stores)
};

// CE, IB, LG from the kind's geometry (shared with the host planner); CH chunks per lane per unit.
template <uint32_t KIND_>
struct Geom {
    static constexpr uint32_t KIND = KIND_, CE = stk::chunk_elems(KIND_), LG = stk::load_word_bytes(KIND_),
                              IB = CE * stk::source_bits(KIND_) / 8;
};

struct KPass : Geom<ST_KIND_PASS_BF16> {
    static constexpr int SCALE = 0;  // no scalar scale
    static constexpr uint32_t CH = stk::kWordsPass;
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e * 2; }
    static __device__ __forceinline__ bool fast(const Ctx&, const uint32_t* in, uint64_t, uint64_t, u32x4* o) {
        o[0] = u32x4{in[0], in[1], in[2], in[3]};
        return true;
    }
};

struct KF16 : Geom<ST_KIND_CAST_F16> {
    static constexpr int SCALE = 0;  // no scalar scale
    static constexpr uint32_t CH = stk::kWordsPass;
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e * 2; }
    static __device__ __forceinline__ bool fast(const Ctx&, const uint32_t* in, uint64_t, uint64_t, u32x4* o) {
        bool nan = false;
#pragma unroll
        for (int k = 0; k < 4; ++k) nan |= (in[k] & 0x7FFFu) > 0x7C00u || (in[k] & 0x7FFF0000u) > 0x7C000000u;
        if (nan) return false;
        uint32_t r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = cvt_bf16x2(h2f(in[k] & 0xFFFFu), h2f(in[k] >> 16));
        o[0] = u32x4{r[0], r[1], r[2], r[3]};
        return true;
    }
};

struct KF32 : Geom<ST_KIND_CAST_F32> {
    static constexpr int SCALE = 0;  // no scalar scale
    static constexpr uint32_t CH = stk::kWordsF32;
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e * 4; }
    static __device__ __forceinline__ bool fast(const Ctx&, const uint32_t* in, uint64_t, uint64_t, u32x4* o) {
        bool nan = false;
#pragma unroll
        for (int k = 0; k < 8; ++k) nan |= (in[k] & 0x7FFFFFFFu) > 0x7F800000u;
        if (nan) return false;
        uint32_t r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = cvt_bf16x2(as_f32(in[2 * k]), as_f32(in[2 * k + 1]));
        o[0] = u32x4{r[0], r[1], r[2], r[3]};
        return true;
    }
};

// 4 e4m3 codes times s -> two packed bf16 pairs
__device__ __forceinline__ void fp8x4_scaled(uint32_t x, float s, uint32_t& lo, uint32_t& hi) {
    const f32x2 a = fp8x2<false>(x), b = fp8x2<true>(x);
    lo = cvt_bf16x2(a.x * s, a.y * s);
    hi = cvt_bf16x2(b.x * s, b.y * s);
}
// 16 e4m3 codes -> two output words; exact path if any code is NaN or s is not finite (so no
// product is NaN)
__device__ __forceinline__ bool fp8_chunk(const uint32_t* in, float s, u32x4* o) {
    const uint32_t t = ((in[0] & 0x7F7F7F7Fu) + 0x01010101u) | ((in[1] & 0x7F7F7F7Fu) + 0x01010101u) |
                       ((in[2] & 0x7F7F7F7Fu) + 0x01010101u) | ((in[3] & 0x7F7F7F7Fu) + 0x01010101u);
    if ((t & 0x80808080u) != 0 || !finite(s)) return false;
    uint32_t r[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) fp8x4_scaled(in[k], s, r[2 * k], r[2 * k + 1]);
    o[0] = u32x4{r[0], r[1], r[2], r[3]};
    o[1] = u32x4{r[4], r[5], r[6], r[7]};
    return true;
}

struct KFp8Tensor : Geom<ST_KIND_FP8_TENSOR> {
    static constexpr int SCALE = 1;  // D.scale
    static constexpr uint32_t CH = stk::kWordsFp8 / 2;
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e; }
    static __device__ __forceinline__ bool fast(const Ctx& c, const uint32_t* in, uint64_t, uint64_t, u32x4* o) {
        return fp8_chunk(in, c.s, o);
    }
};

struct KFp8Block : Geom<ST_KIND_FP8_BLOCK128> {
    static constexpr int SCALE = 0;  // no scalar scale
    static constexpr uint32_t CH = stk::kWordsFp8 / 2;
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e; }
    // e: first output element of the chunk (a multiple of 16); with cols % 16 == 0 the chunk lies
    // in one row and one 128-column block, otherwise it takes the exact path.
    static __device__ __forceinline__ bool fast(const Ctx& c, const uint32_t* in, uint64_t e, uint64_t, u32x4* o) {
        if ((c.D.cols & 15u) != 0) return false;
        const uint32_t e32 = uint32_t(e);
        const uint32_t row = stk::div_apply(e32, c.D.div_magic, c.D.div_shift);
        const uint32_t col = e32 - row * c.D.cols;
        const float S = ld_f32(c.blob + c.D.scale + 4ull * ((row >> 7) * c.D.grid_cols + (col >> 7)), c.scale_al);
        return fp8_chunk(in, S, o);
    }
};

struct KFp4 : Geom<ST_KIND_NVFP4> {
    static constexpr int SCALE = 2;  // D.scale2
    static constexpr uint32_t CH = stk::kWordsFp4;
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e >> 1; }
    // 8 elements from source element x: (e2m1 * block scale) is exact in fp32, then one RNE
    // multiply by g
    static __device__ __forceinline__ bool fast(const Ctx& c, const uint32_t* in, uint64_t, uint64_t xs, u32x4* o) {
        const uint32_t code = ld_u8(c.blob + c.D.scale + (xs >> 4));  // block scale of these 8 elements
        if (!finite(c.s) || (code & 0x7Fu) == 0x7Fu) return false;
        const float bs = fp8x2<false>(code).x;
        const float g = c.s;
        const uint32_t x = in[0];
        const f32x2 p0 = fp4x2<0>(x), p1 = fp4x2<1>(x), p2 = fp4x2<2>(x), p3 = fp4x2<3>(x);
        o[0] = u32x4{cvt_bf16x2((p0.x * bs) * g, (p0.y * bs) * g), cvt_bf16x2((p1.x * bs) * g, (p1.y * bs) * g),
                     cvt_bf16x2((p2.x * bs) * g, (p2.y * bs) * g), cvt_bf16x2((p3.x * bs) * g, (p3.y * bs) * g)};
        return true;
    }
};

static_assert(KPass::IB == 16 && KF32::IB == 32 && KFp8Tensor::IB == 16 && KFp4::IB == 4, "chunk geometry");

// ------------------------------------------------------------------------- loads

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// The IB source bytes of chunk ci (relative to the unit base) as IB/4 dwords in `in`.
//  ALIGNED: base is LG-aligned; IB/LG naturally aligned LG-byte loads.
//  otherwise: base is the 4-byte boundary sh bytes below the source; IB/16 16-byte loads at
//  4-byte alignment (one 4-byte load for NVFP4) plus one trailing dword, then a funnel shift.
template <class K, bool ALIGNED>
struct Fetch {
    static constexpr uint32_t N = K::IB / 4;            // dwords of input per chunk
    static constexpr uint32_t RW = ALIGNED ? N : N + 1;  // dwords loaded per chunk
    static __device__ __forceinline__ void load(const uint8_t* base, uint32_t ci, uint32_t* raw) {
        const uint8_t* p = base + size_t(ci) * K::IB;
        if constexpr (ALIGNED && K::LG == 16) {
#pragma unroll
            for (uint32_t k = 0; k < N / 4; ++k) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(p + 16 * k);
                raw[4 * k] = v.x; raw[4 * k + 1] = v.y; raw[4 * k + 2] = v.z; raw[4 * k + 3] = v.w;
            }
        } else {
            constexpr uint32_t W4 = N / 4;  // 16-byte loads
#pragma unroll
            for (uint32_t k = 0; k < W4; ++k) {
                const u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(p + 16 * k);
                raw[4 * k] = v.x; raw[4 * k + 1] = v.y; raw[4 * k + 2] = v.z; raw[4 * k + 3] = v.w;
            }
#pragma unroll
            for (uint32_t k = 4 * W4; k < RW; ++k) raw[k] = reinterpret_cast<const uint32_t*>(p)[k];
        }
    }
    static __device__ __forceinline__ void align(const uint32_t* raw, uint32_t sh, uint32_t* in) {
#pragma unroll
        for (uint32_t k = 0; k < N; ++k) in[k] = ALIGNED ? raw[k] : __builtin_amdgcn_alignbyte(raw[k + 1], raw[k], sh);
    }
};

// The output pointer and the kind's scalar scale, loaded after the unit's data loads are issued.
// False: the output address is not a bf16 address, and nothing is written.
template <class K>
__device__ __forceinline__ bool finish_ctx(Ctx& c, uint16_t*& out) {
    out = ld_uniform<uint16_t*>(c.outs + c.D.out);
    if constexpr (K::SCALE == 1) c.s = ld_scalar_f32(c.blob + c.D.scale);
    else if constexpr (K::SCALE == 2) c.s = ld_scalar_f32(c.blob + c.D.scale2);
    else c.s = 0.0f;
    const uintptr_t oa = reinterpret_cast<uintptr_t>(out);
    c.vec = (oa & 15u) == 0;
    return (oa & 1u) == 0;
}

// Exact path for one chunk (or its first n elements).
__device__ __forceinline__ void chunk_exact(const Ctx& c, uint16_t* __restrict__ out, uint64_t e, uint32_t n) {
    for (uint32_t k = 0; k < n; ++k) out[e + k] = uint16_t(elem_exact(c.blob, c.D, e + k));
}

// A unit of exactly CH * 64 whole chunks (the default unit size): no per-chunk bounds checks.
template <class K, bool ALIGNED>
__device__ __forceinline__ void unit_full(const Ctx& c0, uint64_t e0, uint32_t sh, uint32_t lane) {
    using F = Fetch<K, ALIGNED>;
    constexpr uint32_t OW = K::CE / stk::kWordElems;
    const uint8_t* base = c0.blob + c0.D.src + K::src_off(e0) - sh;
    uint32_t raw[K::CH][F::RW];
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j) F::load(base, j * stk::kWave + lane, raw[j]);
    Ctx c = c0;
    uint16_t* out;
    if (!finish_ctx<K>(c, out)) return;
    bool ok[K::CH];
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j) {
        uint32_t in[F::N];
        F::align(raw[j], sh, in);
        const uint64_t e = e0 + uint64_t(j * stk::kWave + lane) * K::CE;
        u32x4 v[OW];
        ok[j] = c.vec && K::fast(c, in, e, e, v);
        if (ok[j]) {
#pragma unroll
            for (uint32_t w = 0; w < OW; ++w) *reinterpret_cast<u32x4*>(out + e + w * stk::kWordElems) = v[w];
        }
    }
    bool all = true;
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j) all &= ok[j];
    if (__builtin_amdgcn_ballot_w64(!all) == 0) return;  // the common case
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j)
        if (!ok[j]) chunk_exact(c, out, e0 + uint64_t(j * stk::kWave + lane) * K::CE, K::CE);
}

// Any unit: cnt elements (a larger unit size, or an output's final unit).
template <class K, bool ALIGNED>
__device__ __forceinline__ void unit_any(const Ctx& c0, uint64_t e0, uint32_t cnt, uint32_t sh, uint32_t lane) {
    using F = Fetch<K, ALIGNED>;
    constexpr uint32_t OW = K::CE / stk::kWordElems;
    Ctx c = c0;
    uint16_t* out;
    if (!finish_ctx<K>(c, out)) return;
    const uint8_t* base = c.blob + c.D.src + K::src_off(e0) - sh;
    const uint32_t nch = cnt / K::CE;  // whole chunks
    for (uint32_t ci = lane; ci < nch; ci += stk::kWave) {
        uint32_t raw[F::RW], in[F::N];
        F::load(base, ci, raw);
        F::align(raw, sh, in);
        const uint64_t e = e0 + uint64_t(ci) * K::CE;
        u32x4 v[OW];
        if (c.vec && K::fast(c, in, e, e, v)) {
#pragma unroll
            for (uint32_t w = 0; w < OW; ++w) *reinterpret_cast<u32x4*>(out + e + w * stk::kWordElems) = v[w];
        } else {
            chunk_exact(c, out, e, K::CE);
        }
    }
    for (uint32_t t = nch * K::CE + lane; t < cnt; t += stk::kWave)  // past the last whole chunk
        out[e0 + t] = uint16_t(elem_exact(c.blob, c.D, e0 + t));
}

// A unit of a column slice: chunk starts are mapped to their source elements one by one (the
// host guarantees that a chunk never crosses a row and that every chunk has the alignment of the
// slice's first source byte, or marks the descriptor exact-only).  A whole unit issues all of a
// lane's loads before decoding, like unit_full; a partial one walks its chunks.
template <class K, bool ALIGNED>
__device__ __forceinline__ void unit_strided(const Ctx& c0, uint64_t e0, uint32_t cnt, uint32_t sh, uint32_t lane) {
    using F = Fetch<K, ALIGNED>;
    constexpr uint32_t OW = K::CE / stk::kWordElems;
    const uint8_t* base = c0.blob + c0.D.src - sh;
    if (cnt == K::CE * K::CH * stk::kWave) {
        uint32_t raw[K::CH][F::RW];
        uint64_t xs[K::CH];
#pragma unroll
        for (uint32_t j = 0; j < K::CH; ++j) {
            xs[j] = src_elem(c0.D, e0 + uint64_t(j * stk::kWave + lane) * K::CE);
            F::load(base + K::src_off(xs[j]), 0, raw[j]);
        }
        Ctx c = c0;
        uint16_t* out;
        if (!finish_ctx<K>(c, out)) return;
        bool ok[K::CH];
#pragma unroll
        for (uint32_t j = 0; j < K::CH; ++j) {
            uint32_t in[F::N];
            F::align(raw[j], sh, in);
            const uint64_t e = e0 + uint64_t(j * stk::kWave + lane) * K::CE;
            u32x4 v[OW];
            ok[j] = c.vec && K::fast(c, in, e, xs[j], v);
            if (ok[j]) {
#pragma unroll
                for (uint32_t w = 0; w < OW; ++w) *reinterpret_cast<u32x4*>(out + e + w * stk::kWordElems) = v[w];
            }
        }
        bool all = true;
#pragma unroll
        for (uint32_t j = 0; j < K::CH; ++j) all &= ok[j];
        if (__builtin_amdgcn_ballot_w64(!all) == 0) return;
#pragma unroll
        for (uint32_t j = 0; j < K::CH; ++j)
            if (!ok[j]) chunk_exact(c, out, e0 + uint64_t(j * stk::kWave + lane) * K::CE, K::CE);
        return;
    }
    Ctx c = c0;
    uint16_t* out;
    if (!finish_ctx<K>(c, out)) return;
    const uint32_t nch = cnt / K::CE;
    for (uint32_t ci = lane; ci < nch; ci += stk::kWave) {
        const uint64_t e = e0 + uint64_t(ci) * K::CE;
        const uint64_t x = src_elem(c.D, e);
        uint32_t raw[F::RW], in[F::N];
        F::load(base + K::src_off(x), 0, raw);
        F::align(raw, sh, in);
        u32x4 v[OW];
        if (c.vec && K::fast(c, in, e, x, v)) {
#pragma unroll
            for (uint32_t w = 0; w < OW; ++w) *reinterpret_cast<u32x4*>(out + e + w * stk::kWordElems) = v[w];
        } else {
            chunk_exact(c, out, e, K::CE);
        }
    }
    for (uint32_t t = nch * K::CE + lane; t < cnt; t += stk::kWave)
        out[e0 + t] = uint16_t(elem_exact(c.blob, c.D, e0 + t));
}

template <class K>
__device__ __forceinline__ void run_strided(const Ctx& c, uint64_t e0, uint32_t cnt, uint32_t lane) {
    const uint32_t a = uint32_t(reinterpret_cast<uintptr_t>(c.blob + c.D.src));
    if ((a & (K::LG - 1)) == 0) unit_strided<K, true>(c, e0, cnt, 0, lane);
    else unit_strided<K, false>(c, e0, cnt, a & 3u, lane);
}

// Every element of a unit through the exact path (descriptors the host marks exact-only).
__device__ __forceinline__ void unit_exact(const Ctx& c0, uint64_t e0, uint32_t cnt, uint32_t lane) {
    Ctx c = c0;
    uint16_t* out = ld_uniform<uint16_t*>(c.outs + c.D.out);
    if (reinterpret_cast<uintptr_t>(out) & 1u) return;
    for (uint32_t t = lane; t < cnt; t += stk::kWave) out[e0 + t] = uint16_t(elem_exact(c.blob, c.D, e0 + t));
}

template <class K, bool ALIGNED>
__device__ __forceinline__ void unit_dispatch(const Ctx& c, uint64_t e0, uint32_t cnt, uint32_t sh, uint32_t lane) {
    if (cnt == K::CE * K::CH * stk::kWave) unit_full<K, ALIGNED>(c, e0, sh, lane);
    else unit_any<K, ALIGNED>(c, e0, cnt, sh, lane);
}

// Aligned: the unit's source starts on an LG-byte boundary; otherwise sh = its offset within a
// 4-byte word (0 for a 4-byte-aligned source that is not 16-byte aligned).
template <class K>
__device__ __forceinline__ void run_unit(const Ctx& c, uint64_t e0, uint32_t cnt, uint32_t lane) {
    const uint32_t a = uint32_t(reinterpret_cast<uintptr_t>(c.blob + c.D.src + K::src_off(e0)));
    if ((a & (K::LG - 1)) == 0) unit_dispatch<K, true>(c, e0, cnt, 0, lane);
    else unit_dispatch<K, false>(c, e0, cnt, a & 3u, lane);
}

// ------------------------------------------------------------------------- the kernel

// SLICES: the instance that runs column slices through the strided fast path.  The plain instance
// sends them (and exact-only descriptors) through the per-element exact path; keeping the strided
// code out of it was measured to matter (2-5% on the whole-checkpoint decode).
template <bool SLICES>
__global__ __launch_bounds__(kBlock) void materialize_kernel(const uint8_t* __restrict__ blob,
                                                             const uint8_t* __restrict__ table, uint32_t units,
                                                             uint32_t groups, uint32_t desc_off,
                                                             uint16_t* const* __restrict__ outs) {
    // XCD-contiguous renumbering: workgroup b runs on XCD b % 8; XCD x gets the contiguous range
    // of groups [start_x, start_x + count_x), a bijection of [0, groups).
    const uint32_t b = blockIdx.y * gridDim.x + blockIdx.x;
    if (b >= groups) return;
    const uint32_t x = b & 7u, q = groups >> 3, rem = groups & 7u;
    const uint32_t grp = x * q + (x < rem ? x : rem) + (b >> 3);
    const uint32_t unit = grp * ST_UNITS_PER_GROUP + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (unit >= units) return;
    const uint32_t lane = threadIdx.x & (stk::kWave - 1);

    // Header (magic, unit count), this group's map entry, then the descriptor: the only loads
    // ahead of the data.  A table that does not match n is left alone before anything indexes it.
    const u32x4 hw = ld_uniform<u32x4>(table);
    if ((hw.x != ST_TABLE_MAGIC) | (hw.z != units) | (hw.w != 0)) return;
    uint32_t d = ld_uniform<uint32_t>(table + sizeof(st_table_header) + 4 * size_t(grp));
    const st_desc* descs = reinterpret_cast<const st_desc*>(table + desc_off);
    Desc D = load_desc(descs + d);
    while (unit >= D.unit_end) D = load_desc(descs + (++d));  // at most 3 steps, past empty outputs

    const uint64_t e0 = uint64_t(unit - D.unit_begin) << D.unit_shift;
    const uint32_t cnt = unit + 1 == D.unit_end ? D.tail : 1u << D.unit_shift;
    Ctx c;
    c.blob = blob;
    c.D = D;
    c.outs = outs;
    c.scale_al = (D.scale & 3u) == 0;
    if ((D.pitch | D.flags) != 0) {  // column slices and exact-only descriptors
        if (!SLICES || (D.flags & ST_DESC_EXACT)) {
            unit_exact(c, e0, cnt, lane);
            return;
        }
        switch (D.kind) {
            case ST_KIND_FP8_TENSOR: run_strided<KFp8Tensor>(c, e0, cnt, lane); break;
            case ST_KIND_FP8_BLOCK128: run_strided<KFp8Block>(c, e0, cnt, lane); break;
            case ST_KIND_NVFP4: run_strided<KFp4>(c, e0, cnt, lane); break;
            case ST_KIND_PASS_BF16: run_strided<KPass>(c, e0, cnt, lane); break;
            case ST_KIND_CAST_F16: run_strided<KF16>(c, e0, cnt, lane); break;
            default: run_strided<KF32>(c, e0, cnt, lane); break;
        }
        return;
    }
    switch (D.kind) {
        case ST_KIND_FP8_TENSOR: run_unit<KFp8Tensor>(c, e0, cnt, lane); break;
        case ST_KIND_FP8_BLOCK128: run_unit<KFp8Block>(c, e0, cnt, lane); break;
        case ST_KIND_NVFP4: run_unit<KFp4>(c, e0, cnt, lane); break;
        case ST_KIND_PASS_BF16: run_unit<KPass>(c, e0, cnt, lane); break;
        case ST_KIND_CAST_F16: run_unit<KF16>(c, e0, cnt, lane); break;
        default: run_unit<KF32>(c, e0, cnt, lane); break;
    }
}

template <bool SLICES>
st_status launch(const char* who, const void* blob, const void* descs, size_t n, void* const* outs, void* stream) {
    if (n == 0) return ST_OK;
    if (!blob || !descs || !outs) return st_fail(ST_E_ARG, "%s: null pointer", who);
    if (reinterpret_cast<uintptr_t>(blob) % ST_BLOB_ALIGN)
        return st_fail(ST_E_ARG, "%s: blob is not %d-byte aligned", who, ST_BLOB_ALIGN);
    if (reinterpret_cast<uintptr_t>(descs) % 64) return st_fail(ST_E_ARG, "%s: work table is not 64-byte aligned", who);
    if (uint64_t(n) >= (uint64_t(1) << 32)) return st_fail(ST_E_ARG, "%s: %zu work units (at most 2^32 - 1)", who, n);
    const uint32_t groups = uint32_t((uint64_t(n) + ST_UNITS_PER_GROUP - 1) / ST_UNITS_PER_GROUP);
    const uint32_t gx = groups < kMaxGridX ? groups : kMaxGridX;
    const uint32_t gy = (groups + gx - 1) / gx;
    hipLaunchKernelGGL(materialize_kernel<SLICES>, dim3(gx, gy), dim3(kBlock), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint8_t*>(blob), static_cast<const uint8_t*>(descs), uint32_t(n), groups,
                       uint32_t(stk::table_desc_offset(groups)), reinterpret_cast<uint16_t* const*>(outs));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return st_fail(ST_E_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return ST_OK;
}

}  // namespace

extern "C" st_status st_materialize(const void* blob, const void* descs, size_t n, void* const* outs, void* stream) {
    return launch<false>("st_materialize", blob, descs, n, outs, stream);
}

extern "C" st_status st_materialize_slices(const void* blob, const void* descs, size_t n, void* const* outs,
                                           void* stream) {
    return launch<true>("st_materialize_slices", blob, descs, n, outs, stream);
}
