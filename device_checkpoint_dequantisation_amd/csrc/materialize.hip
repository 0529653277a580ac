// The grouped materialise kernel: one launch turns every descriptor's bytes in the device blob
// into bf16 outputs (or fp16 / fp32 outputs, one kernel instance per output type).
//
// What it computes is fixed by the checkpoint formats the pages name ("Resident Modal LLM
// Architecture", "Current Backend Boundary": Qwen block-FP8, ModelOpt NVFP4; "Disk tier
// safetensors streaming design audit", "Mandatory research audit": ComfyUI scaled FP8), plus the
// OCP Microscaling formats MXFP8 / MXFP4 (E8M0 scale per 32 elements), read as OCP E4M3 /
// OCP-MX E2M1 codes, one IEEE binary32 round-to-nearest-even multiply per scale and a
// round-to-nearest-even narrowing to the output type (bfloat16 by default; NaN -> the type's
// canonical quiet NaN; no subnormal flushing).  A bf16 source copied to a bf16 output keeps its
// bits.
//
// Shape of the work.  This is a memory-bound elementwise codec (2.6-6 bytes of HBM traffic per
// element, a handful of VALU operations per element), so there is no matrix-core work; what
// matters on gfx950 is how the HBM traffic is issued:
//  * One wavefront per work unit, one-shot.  A unit is 512-2048 elements of one output (about
//    0.5-2 KB read, 1-4 KB written; measured best against half and double sizes).  Each
//    wavefront loads its unit, decodes, stores and exits.
//    Measured on MI355X, one-shot wavefronts sustain ~20% more read+write bandwidth than any
//    persistent loop tried (grid-stride, contiguous ranges, software-pipelined), because a
//    persistent wavefront's next loads wait behind its own outstanding stores (vmcnt counts both).
//  * Lane-contiguous chunks.  A chunk is one 16-byte output word: 8 elements of a 2-byte output
//    type, 4 of fp32 (packed fp4 keeps 8-element chunks and pairs lanes instead: see
//    unit_full_paired).  Chunk j*64 + l of a unit belongs to lane l, so a store instruction of a
//    wavefront covers 1 KB of contiguous output and a load instruction a contiguous run of the
//    source; lanes read whatever input bytes their chunk needs (4, 8 or 16 bytes; 32 for fp32
//    sources to 2-byte outputs).  Measured on MI355X, lanes that each store two adjacent words
//    lose about 20%, four adjacent words about 30%.
//  * XCD-contiguous order.  The hardware hands workgroup b to XCD b mod 8; workgroups are
//    renumbered so each XCD streams through one contiguous eighth of the work (the host planner
//    balances the eighths' bytes when formats of different bytes per unit mix).
//  * Tiny tensors.  Units are numbered consecutively across outputs and a workgroup's four
//    wavefronts take four consecutive units, whatever output they belong to, so small tensors are
//    packed at wavefront granularity.  A per-workgroup map gives the descriptor of the group's
//    first unit; a wavefront walks forward from it (at most three descriptors, plus any outputs
//    with no units in between).
//  * Unaligned sources.  A tensor may start at any byte.  A unit whose source is aligned to its
//    chunk's load word (the chunk's source bytes, at most 16) loads whole words.  Otherwise each lane
//    loads from the 4-byte boundary at or below its bytes (16-byte words at 4-byte alignment and
//    one load of the remaining dwords, one more dword than the chunk needs), and the byte offset
//    sh (the same for every lane of a unit) is removed in registers with v_alignbyte.  Measured
//    on MI355X, this beats loading the two enclosing aligned words and selecting among them.
//  * Short dependency chain.  Ahead of a wavefront's data loads sit only the table header check,
//    its map entry and its descriptor; the output pointer and the scalar scale are loaded once the
//    data loads are in flight (a wait for one scalar load waits for all of them), and no branch
//    on those values or on a block scale precedes the decode (see unit_full).
//  * Decoding uses gfx950's conversion instructions (fp8 and fp4 to fp32, fp32 to bf16 and to
//    fp16), each checked exhaustively against the exact decoding on the device; one fp32 multiply
//    per scale.
//  * Tails, NaN inputs, non-finite scales, block-FP8 widths not a multiple of 8 and misaligned
//    outputs go through an exact per-element path written from the definitions alone.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstring>
#include <mutex>

#include "st_internal.h"

// Device storage of st_materialize_noalloc: the work table and the output-pointer array of the
// latest call on each GPU (every GPU the library runs on holds its own copy until the process ends).
// Host code never names it directly: its per-device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[ST_NOALLOC_SCRATCH_BYTES];

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// A 16-byte word through an explicitly global pointer.
typedef __attribute__((address_space(1))) u32x4 global_u32x4;
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

// fp16 bits of f rounded to nearest, ties to even, from the IEEE definition (NaN -> 0x7E00;
// subnormal results kept; magnitudes from 65520 up -> infinity).  Below 2^-14 the fp16 code is
// |f| / 2^-24 rounded to an integer: |f| * 2^24 is exact and below 2^10, and adding then
// subtracting 2^23 rounds it to nearest even in binary32 (a code of 1024 is the smallest normal).
__device__ __forceinline__ uint32_t f16_canon(float f) {
    const uint32_t u = as_u32(f), sign = (u >> 16) & 0x8000u, a = u & 0x7FFFFFFFu;
    if (a > 0x7F800000u) return 0x7E00u;
    if (a >= 0x477FF000u) return sign | 0x7C00u;
    if (a < 0x38800000u) {
        const float y = as_f32(a) * 16777216.0f + 8388608.0f;
        return sign | uint32_t(y - 8388608.0f);
    }
    const uint32_t t = a + 0xFFFu + ((a >> 13) & 1u);
    return sign | ((t >> 13) - (112u << 10));
}
__device__ __forceinline__ uint32_t f32_canon(float f) { return f != f ? 0x7FC00000u : as_u32(f); }

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
// E8M0 scale code -> 2^(c - 127) as binary32: exponent field c, or for c = 0 the subnormal 2^-127
// (mantissa bit 22); 0xFF is NaN.  Used on both paths: the value is exact either way.
__device__ __forceinline__ float e8m0_exact(uint32_t c) {
    return c == 0xFFu ? __builtin_nanf("") : as_f32(c != 0 ? c << 23 : 0x00400000u);
}

// True if any byte of x is an e4m3 NaN code (0x7F or 0xFF).
__device__ __forceinline__ bool has_nan_code(uint32_t x) {
    return (((x & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u) != 0;
}

// gfx950 conversion instructions used on the fast path.  Each was checked exhaustively on the
// device against the exact decoding above: v_cvt_pk_f32_fp8 on every pair of e4m3 codes (it
// decodes OCP e4m3fn), v_cvt_scalef32_pk_f32_fp4 with scale 1.0 on every byte, and
// v_cvt_pk_bf16_f32 and v_cvt_pk_f16_f32 on all 2^32 fp32 patterns (round to nearest even,
// subnormals kept; both keep NaN payloads, so the fast path never hands them a NaN).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t cvt_bf16x2(float a, float b) {  // a at the lower address
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ uint32_t cvt_f16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}
// e4m3 codes in bytes 0,1 (HI: 2,3) of x -> exact fp32 values
template <bool HI>
__device__ __forceinline__ f32x2 fp8x2(uint32_t x) { return __builtin_amdgcn_cvt_pk_f32_fp8(x, HI); }
// e2m1 codes in byte P of x (low nibble first) -> exact fp32 values
template <int P>
__device__ __forceinline__ f32x2 fp4x2(uint32_t x) { return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, P); }
__device__ __forceinline__ bool finite(float s) { return __builtin_fabsf(s) <= 3.4028234663852886e38f; }

// ------------------------------------------------------------------------- output types
//
// An output type turns fp32 results into output bits: pack2 on the fast path (inputs never NaN),
// exact on the exact path.  BYTES per element; CODE is the st_out_dtype the work table records.

struct OutBf16 {
    static constexpr uint32_t BYTES = 2, CODE = ST_OUT_BF16;
    static __device__ __forceinline__ uint32_t pack2(float a, float b) { return cvt_bf16x2(a, b); }
    static __device__ __forceinline__ uint32_t exact(float f) { return bf16_canon(f); }
};
struct OutF16 {
    static constexpr uint32_t BYTES = 2, CODE = ST_OUT_F16;
    static __device__ __forceinline__ uint32_t pack2(float a, float b) { return cvt_f16x2(a, b); }
    static __device__ __forceinline__ uint32_t exact(float f) { return f16_canon(f); }
};
struct OutF32 {
    static constexpr uint32_t BYTES = 4, CODE = ST_OUT_F32;
    static __device__ __forceinline__ uint32_t exact(float f) { return f32_canon(f); }
};
// An output type with the kernel instance's store policy: NT, non-temporal 16-byte output stores
// (ST_MAT_STREAM_STORES).  A compile-time constant: a run-time choice between the two stores does
// not survive compilation, as the compiler merges them into one plain store.
template <class Base, bool NT_>
struct Stored : Base {
    static constexpr bool NT = NT_;
};

// Output words of a chunk: pair k of values goes to word k (2-byte types) or words 2k, 2k+1.
template <class O>
__device__ __forceinline__ void put2(uint32_t* w, uint32_t k, float a, float b) {
    if constexpr (O::BYTES == 2) {
        w[k] = O::pack2(a, b);
    } else {
        w[2 * k] = as_u32(a);
        w[2 * k + 1] = as_u32(b);
    }
}

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
// row * pitch + col of the slice's source rows, with row = e / cols and col = e % cols.  A split
// descriptor reads its rows whole (e is the source element; its destination is split_dst).
__device__ __forceinline__ uint64_t src_elem(const Desc& D, uint64_t e) {
    if (D.pitch == 0 || (D.flags & ST_DESC_SPLIT)) return e;
    const uint32_t row = stk::div_apply(uint32_t(e), D.div_magic, D.div_shift);
    return e + uint64_t(row) * (D.pitch - D.cols);
}

// Destination of source element e of a split descriptor: the rows [pitch] are cut into 2^grid_cols
// shards of cols elements each; shard s = (e / cols) mod 2^grid_cols is output out + s, a
// [rows, cols] row-major array, and e lands at (e / pitch) * cols + e mod cols in it.  Returns the
// element index; *which = s.
__device__ __forceinline__ uint32_t split_dst(const Desc& D, uint64_t e, uint32_t* which) {
    const uint32_t q = stk::div_apply(uint32_t(e), D.div_magic, D.div_shift);
    *which = q & ((1u << D.grid_cols) - 1u);
    return (q >> D.grid_cols) * D.cols + (uint32_t(e) - q * D.cols);
}

// The exact fp32 value of element e of a KIND descriptor (before the output rounding), straight
// from the definition, byte by byte.
template <uint32_t KIND>
__device__ __forceinline__ float kind_value(const uint8_t* __restrict__ blob, const Desc& D, uint64_t e) {
    const uint8_t* s = blob + D.src;
    const uint64_t x = src_elem(D, e);
    if constexpr (KIND == ST_KIND_PASS_BF16) {
        return as_f32(ld_u16_any(s + 2 * x) << 16);
    } else if constexpr (KIND == ST_KIND_CAST_F16) {
        return h2f(ld_u16_any(s + 2 * x));
    } else if constexpr (KIND == ST_KIND_CAST_F32) {
        return as_f32(ld_u32_any(s + 4 * x));
    } else if constexpr (KIND == ST_KIND_FP8_TENSOR) {
        return e4m3_exact(ld_u8(s + x)) * as_f32(ld_u32_any(blob + D.scale));
    } else if constexpr (KIND == ST_KIND_FP8_BLOCK128) {  // scale grid position from the output's row and column
        const uint32_t e32 = uint32_t(e);
        const uint32_t row = stk::div_apply(e32, D.div_magic, D.div_shift);
        const uint32_t col = e32 - row * D.cols;
        const float S = as_f32(ld_u32_any(blob + D.scale + 4ull * ((row >> 7) * D.grid_cols + (col >> 7))));
        return e4m3_exact(ld_u8(s + x)) * S;
    } else if constexpr (KIND == ST_KIND_NVFP4) {  // K % 16 == 0: block scale (i, j / 16) at flat index x / 16
        const uint32_t nib = (ld_u8(s + (x >> 1)) >> ((x & 1) * 4)) & 15u;
        const float bs = e4m3_exact(ld_u8(blob + D.scale + (x >> 4)));
        const float g = as_f32(ld_u32_any(blob + D.scale2));
        const float t = e2m1_exact(nib) * bs;
        return t * g;
    } else {  // MXFP8 / MXFP4: K % 32 == 0: scale (i, j / 32) at flat index x / 32
        static_assert(KIND == ST_KIND_MXFP8 || KIND == ST_KIND_MXFP4, "kind");
        const float S = e8m0_exact(ld_u8(blob + D.scale + (x >> 5)));
        if constexpr (KIND == ST_KIND_MXFP8) return e4m3_exact(ld_u8(s + x)) * S;
        else return e2m1_exact((ld_u8(s + (x >> 1)) >> ((x & 1) * 4)) & 15u) * S;
    }
}

// Output bits of element e of a KIND descriptor: a bf16 source to a bf16 output keeps its bits;
// everything else is the exact value rounded to the output type.
template <uint32_t KIND, class O>
__device__ __forceinline__ uint32_t kind_exact(const uint8_t* __restrict__ blob, const Desc& D, uint64_t e) {
    if constexpr (O::CODE == ST_OUT_BF16 && KIND == ST_KIND_PASS_BF16) return ld_u16_any(blob + D.src + 2 * src_elem(D, e));
    else return O::exact(kind_value<KIND>(blob, D, e));
}

template <class O>
__device__ __forceinline__ void store_elem(uint8_t* out, uint64_t e, uint32_t bits) {
    if constexpr (O::BYTES == 2) reinterpret_cast<uint16_t*>(out)[e] = uint16_t(bits);
    else reinterpret_cast<uint32_t*>(out)[e] = bits;
}

// ------------------------------------------------------------------------- per-kind chunks
//
// A Kind decodes one chunk of CE elements from IB input bytes, fetched as naturally aligned
// LG-byte words, into CE * O::BYTES / 4 output words.  `sc` loads the chunk's scale word (a scale
// code, or an fp32 scale's bits; 0 for kinds without a per-chunk scale) from the chunk's output
// element e and source element xs; `fast` decodes with it and returns false when the chunk must
// take the exact path.  CH = chunks per lane per unit; chunk c of a unit belongs to lane c % 64.
// Kinds with a per-chunk scale (SC_LOAD) load it either together with the data, before the first
// store (EARLY_SC), or just before the chunk's decode, behind a scheduling barrier so that the load
// is issued before the decode waits for the chunk's data.  Measured on MI355X: loading early gains
// about 1% for block FP8 into 2-byte outputs and loses 0.5-1.5% for the others (single-byte scale
// codes that mostly hit in cache); letting the compiler place the late load after the data wait
// cost MXFP8 3%.  Whole units of packed fp4 fetch all their codes at once instead (UnitCodes).

// Per-unit context.  `s` and `vec` are filled in by finish_ctx, after the data loads are issued;
// whether the scale folds into the fast path is decided in the decode.
struct Ctx {
    const uint8_t* blob;
    Desc D;
    uint8_t* const* outs;  // output pointers, indexed by the descriptor's `out`
    float s;         // FP8_TENSOR: the per-tensor scale; NVFP4: the global scale
    bool scale_al;   // the descriptor's scale data is 4-byte aligned
    bool vec;        // the output is 16-byte aligned (vector stores)
};

// Chunk geometry of kind KIND_ for output type O.  A chunk is one 16-byte output word: 8 elements
// of a 2-byte type, or 4 elements of fp32, so that a store instruction of a wavefront covers
// contiguous output for every output type (measured on MI355X: lanes storing two adjacent fp32
// words lose about 20%).  Packed fp4 keeps 8-element chunks for fp32 too (4-byte loads).  IB
// source bytes per chunk, loaded as naturally aligned LG-byte words (IB, at most 16); N = IB / 4
// dwords; CH chunks per lane in a unit of the default size.  For 2-byte outputs CE and LG are the
// host planner's chunk_elems and load_word_bytes, whose column-slice rules are therefore also
// sufficient for the 4-element fp32 chunks.
template <uint32_t KIND_, class O>
struct Geom {
    static constexpr bool FP4 = KIND_ == ST_KIND_NVFP4 || KIND_ == ST_KIND_MXFP4;
    static constexpr uint32_t KIND = KIND_, CE = (O::BYTES == 4 && !FP4) ? 4 : 8,
                              IB = CE * stk::source_bits(KIND_) / 8, LG = IB < 16 ? IB : 16, N = IB / 4,
                              CH = stk::words_per_lane(KIND_, O::CODE) * stk::kWordElems / CE;
    // whole units of packed fp4 into fp32 take unit_full_paired
    static constexpr bool PAIRED = FP4 && O::BYTES == 4;
    static constexpr bool SC_LOAD = KIND_ == ST_KIND_FP8_BLOCK128 || KIND_ == ST_KIND_NVFP4 || KIND_ == ST_KIND_MXFP8 ||
                                    KIND_ == ST_KIND_MXFP4;
    static constexpr bool EARLY_SC = false;
    // Packed fp4 whole units (unit_full, unit_full_paired) fetch their scale codes once per unit
    // (UnitCodes); the elements one code covers, 0 for the other kinds
    static constexpr uint32_t UNIT_SB = KIND_ == ST_KIND_NVFP4 ? 16 : KIND_ == ST_KIND_MXFP4 ? 32 : 0;
    static_assert(O::BYTES == 4 || (CE == stk::chunk_elems(KIND_) && LG == stk::load_word_bytes(KIND_)),
                  "2-byte outputs use the host planner's geometry");
};

template <class O>
struct KPass : Geom<ST_KIND_PASS_BF16, O> {
    using G = Geom<ST_KIND_PASS_BF16, O>;
    static constexpr int SCALE = 0;  // no scalar scale
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e * 2; }
    static __device__ __forceinline__ uint32_t sc(const Ctx&, uint64_t, uint64_t) { return 0; }
    static __device__ __forceinline__ bool fast(const Ctx&, const uint32_t* in, uint32_t, uint32_t* w) {
        if constexpr (O::CODE == ST_OUT_BF16) {  // the bits themselves
#pragma unroll
            for (uint32_t k = 0; k < G::N; ++k) w[k] = in[k];
            return true;
        } else {
            bool nan = false;
#pragma unroll
            for (uint32_t k = 0; k < G::N; ++k)
                nan |= (in[k] & 0x7FFFu) > 0x7F80u || (in[k] & 0x7FFF0000u) > 0x7F800000u;
#pragma unroll
            for (uint32_t k = 0; k < G::N; ++k) put2<O>(w, k, as_f32(in[k] << 16), as_f32(in[k] & 0xFFFF0000u));
            return !nan;
        }
    }
};

template <class O>
struct KF16 : Geom<ST_KIND_CAST_F16, O> {
    using G = Geom<ST_KIND_CAST_F16, O>;
    static constexpr int SCALE = 0;  // no scalar scale
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e * 2; }
    static __device__ __forceinline__ uint32_t sc(const Ctx&, uint64_t, uint64_t) { return 0; }
    static __device__ __forceinline__ bool fast(const Ctx&, const uint32_t* in, uint32_t, uint32_t* w) {
        bool nan = false;
#pragma unroll
        for (uint32_t k = 0; k < G::N; ++k) nan |= (in[k] & 0x7FFFu) > 0x7C00u || (in[k] & 0x7FFF0000u) > 0x7C000000u;
#pragma unroll
        for (uint32_t k = 0; k < G::N; ++k) {
            if constexpr (O::CODE == ST_OUT_F16) w[k] = in[k];  // fp16 to fp16: the value is exact
            else put2<O>(w, k, h2f(in[k] & 0xFFFFu), h2f(in[k] >> 16));
        }
        return !nan;
    }
};

template <class O>
struct KF32 : Geom<ST_KIND_CAST_F32, O> {
    using G = Geom<ST_KIND_CAST_F32, O>;
    static constexpr int SCALE = 0;  // no scalar scale
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e * 4; }
    static __device__ __forceinline__ uint32_t sc(const Ctx&, uint64_t, uint64_t) { return 0; }
    static __device__ __forceinline__ bool fast(const Ctx&, const uint32_t* in, uint32_t, uint32_t* w) {
        bool nan = false;
#pragma unroll
        for (uint32_t k = 0; k < G::N; ++k) nan |= (in[k] & 0x7FFFFFFFu) > 0x7F800000u;
#pragma unroll
        for (uint32_t k = 0; k < G::N / 2; ++k) put2<O>(w, k, as_f32(in[2 * k]), as_f32(in[2 * k + 1]));
        return !nan;
    }
};

// 4N e4m3 codes times s -> output words; exact path if any code is NaN or s is not finite (so no
// product is NaN)
template <class O, uint32_t N>
__device__ __forceinline__ bool fp8_chunk(const uint32_t* in, float s, uint32_t* w) {
    uint32_t t = 0;
#pragma unroll
    for (uint32_t k = 0; k < N; ++k) t |= (in[k] & 0x7F7F7F7Fu) + 0x01010101u;
#pragma unroll
    for (uint32_t k = 0; k < N; ++k) {
        const f32x2 a = fp8x2<false>(in[k]), b = fp8x2<true>(in[k]);
        put2<O>(w, 2 * k, a.x * s, a.y * s);
        put2<O>(w, 2 * k + 1, b.x * s, b.y * s);
    }
    return ((t & 0x80808080u) == 0) & finite(s);
}

template <class O>
struct KFp8Tensor : Geom<ST_KIND_FP8_TENSOR, O> {
    using G = Geom<ST_KIND_FP8_TENSOR, O>;
    static constexpr int SCALE = 1;  // D.scale
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e; }
    static __device__ __forceinline__ uint32_t sc(const Ctx&, uint64_t, uint64_t) { return 0; }
    static __device__ __forceinline__ bool fast(const Ctx& c, const uint32_t* in, uint32_t, uint32_t* w) {
        return fp8_chunk<O, G::N>(in, c.s, w);
    }
};

template <class O>
struct KFp8Block : Geom<ST_KIND_FP8_BLOCK128, O> {
    using G = Geom<ST_KIND_FP8_BLOCK128, O>;
    static constexpr int SCALE = 0;  // no scalar scale
    static constexpr bool EARLY_SC = O::BYTES == 2;
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e; }
    // e: first output element of the chunk (a multiple of CE); with cols % CE == 0 the chunk lies
    // in one row and one 128-column block, otherwise it takes the exact path.
    static __device__ __forceinline__ uint32_t sc(const Ctx& c, uint64_t e, uint64_t) {
        if ((c.D.cols & (G::CE - 1)) != 0) return 0;
        const uint32_t e32 = uint32_t(e);
        const uint32_t row = stk::div_apply(e32, c.D.div_magic, c.D.div_shift);
        const uint32_t col = e32 - row * c.D.cols;
        return as_u32(ld_f32(c.blob + c.D.scale + 4ull * ((row >> 7) * c.D.grid_cols + (col >> 7)), c.scale_al));
    }
    static __device__ __forceinline__ bool fast(const Ctx& c, const uint32_t* in, uint32_t sc, uint32_t* w) {
        return ((c.D.cols & (G::CE - 1)) == 0) & fp8_chunk<O, G::N>(in, as_f32(sc), w);
    }
};

template <class O>
struct KFp4 : Geom<ST_KIND_NVFP4, O> {
    static constexpr int SCALE = 2;  // D.scale2
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e >> 1; }
    // 8 elements from source element xs: (e2m1 * block scale) is exact in fp32, then one RNE
    // multiply by g
    // the e4m3 block scale of the chunk's 16-element block
    static __device__ __forceinline__ uint32_t sc(const Ctx& c, uint64_t, uint64_t xs) {
        return ld_u8(c.blob + c.D.scale + (xs >> 4));
    }
    static __device__ __forceinline__ bool fast(const Ctx& c, const uint32_t* in, uint32_t code, uint32_t* w) {
        const float bs = fp8x2<false>(code).x;
        const float g = c.s;
        const uint32_t x = in[0];
        const f32x2 p0 = fp4x2<0>(x), p1 = fp4x2<1>(x), p2 = fp4x2<2>(x), p3 = fp4x2<3>(x);
        put2<O>(w, 0, (p0.x * bs) * g, (p0.y * bs) * g);
        put2<O>(w, 1, (p1.x * bs) * g, (p1.y * bs) * g);
        put2<O>(w, 2, (p2.x * bs) * g, (p2.y * bs) * g);
        put2<O>(w, 3, (p3.x * bs) * g, (p3.y * bs) * g);
        return finite(g) & ((code & 0x7Fu) != 0x7Fu);  // decided last: see unit_full
    }
    // 4 elements from bytes B and B + 1 of x, with their block's scale code (unit_full_paired)
    template <int B>
    static __device__ __forceinline__ bool quad(const Ctx& c, uint32_t x, uint32_t code, uint32_t* w) {
        const float bs = fp8x2<false>(code).x;
        const float g = c.s;
        const f32x2 p0 = fp4x2<B>(x), p1 = fp4x2<B + 1>(x);
        put2<O>(w, 0, (p0.x * bs) * g, (p0.y * bs) * g);
        put2<O>(w, 1, (p1.x * bs) * g, (p1.y * bs) * g);
        return finite(g) & ((code & 0x7Fu) != 0x7Fu);
    }
};

// OCP Microscaling: the chunk's elements from source element xs (a multiple of the chunk size)
// share the E8M0 scale of their 32-element block, applied by one RNE multiply; an NaN scale or
// element code takes the exact path.
template <class O>
struct KMx8 : Geom<ST_KIND_MXFP8, O> {
    using G = Geom<ST_KIND_MXFP8, O>;
    static constexpr int SCALE = 0;  // no scalar scale
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e; }
    static __device__ __forceinline__ uint32_t sc(const Ctx& c, uint64_t, uint64_t xs) {
        return ld_u8(c.blob + c.D.scale + (xs >> 5));
    }
    static __device__ __forceinline__ bool fast(const Ctx& c, const uint32_t* in, uint32_t code, uint32_t* w) {
        return fp8_chunk<O, G::N>(in, e8m0_exact(code), w);  // a NaN scale code fails its finite check
    }
};

template <class O>
struct KMx4 : Geom<ST_KIND_MXFP4, O> {
    static constexpr int SCALE = 0;  // no scalar scale
    static __device__ __forceinline__ uint64_t src_off(uint64_t e) { return e >> 1; }
    static __device__ __forceinline__ uint32_t sc(const Ctx& c, uint64_t, uint64_t xs) {
        return ld_u8(c.blob + c.D.scale + (xs >> 5));
    }
    static __device__ __forceinline__ bool fast(const Ctx& c, const uint32_t* in, uint32_t code, uint32_t* w) {
        const float S = e8m0_exact(code);
        const uint32_t x = in[0];
        const f32x2 p0 = fp4x2<0>(x), p1 = fp4x2<1>(x), p2 = fp4x2<2>(x), p3 = fp4x2<3>(x);
        put2<O>(w, 0, p0.x * S, p0.y * S);
        put2<O>(w, 1, p1.x * S, p1.y * S);
        put2<O>(w, 2, p2.x * S, p2.y * S);
        put2<O>(w, 3, p3.x * S, p3.y * S);
        return code != 0xFFu;  // decided last: see unit_full
    }
    // 4 elements from bytes B and B + 1 of x, with their block's scale code (unit_full_paired)
    template <int B>
    static __device__ __forceinline__ bool quad(const Ctx&, uint32_t x, uint32_t code, uint32_t* w) {
        const float S = e8m0_exact(code);
        const f32x2 p0 = fp4x2<B>(x), p1 = fp4x2<B + 1>(x);
        put2<O>(w, 0, p0.x * S, p0.y * S);
        put2<O>(w, 1, p1.x * S, p1.y * S);
        return code != 0xFFu;
    }
};

static_assert(KPass<OutBf16>::IB == 16 && KF32<OutBf16>::IB == 32 && KFp8Tensor<OutBf16>::IB == 8 &&
                  KFp4<OutBf16>::IB == 4 && KMx8<OutBf16>::IB == 8 && KMx4<OutBf16>::IB == 4,
              "chunk geometry, 2-byte outputs");
static_assert(KPass<OutF32>::IB == 8 && KF32<OutF32>::IB == 16 && KFp8Tensor<OutF32>::IB == 4 &&
                  KFp4<OutF32>::IB == 4 && KFp8Tensor<OutF32>::CH == 2 * stk::kWordsFp8,
              "chunk geometry, fp32 outputs");

// ------------------------------------------------------------------------- loads

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));

// The IB source bytes of chunk ci (relative to the unit base) as IB/4 dwords in `in`.
//  ALIGNED: base is LG-aligned (LG = IB except for 32-byte fp32 chunks: two 16-byte words);
//  naturally aligned loads.
//  otherwise: base is the 4-byte boundary sh bytes below the source; the IB bytes plus one
//  trailing dword as 16-byte loads at 4-byte alignment and one load of the remaining 1-3 dwords,
//  then a funnel shift.
// A load of *p, non-temporal (nt) if NTL.
template <bool NTL, class T>
__device__ __forceinline__ T ld(const T* p) {
    if constexpr (NTL) return __builtin_nontemporal_load(p);
    else return *p;
}

template <class K, bool ALIGNED>
struct Fetch {
    static constexpr uint32_t N = K::IB / 4;            // dwords of input per chunk
    static constexpr uint32_t RW = ALIGNED ? N : N + 1;  // dwords loaded per chunk
    // NTL: non-temporal loads (the column-slice path's per-lane addresses)
    template <bool NTL = false>
    static __device__ __forceinline__ void load(const uint8_t* base, uint32_t ci, uint32_t* raw) {
        const uint8_t* p = base + size_t(ci) * K::IB;
        if constexpr (ALIGNED && K::LG == 16) {
#pragma unroll
            for (uint32_t k = 0; k < N / 4; ++k) {
                const u32x4 v = ld<NTL>(reinterpret_cast<const u32x4*>(p + 16 * k));
                raw[4 * k] = v.x; raw[4 * k + 1] = v.y; raw[4 * k + 2] = v.z; raw[4 * k + 3] = v.w;
            }
        } else if constexpr (ALIGNED && K::LG == 8) {
            const u32x2 v = ld<NTL>(reinterpret_cast<const u32x2*>(p));
            raw[0] = v.x; raw[1] = v.y;
        } else if constexpr (ALIGNED) {
            raw[0] = ld<NTL>(reinterpret_cast<const uint32_t*>(p));
        } else {
            constexpr uint32_t W4 = RW / 4, R = RW - 4 * W4;  // 16-byte loads, then R dwords
#pragma unroll
            for (uint32_t k = 0; k < W4; ++k) {
                const u32x4_a4 v = ld<NTL>(reinterpret_cast<const u32x4_a4*>(p + 16 * k));
                raw[4 * k] = v.x; raw[4 * k + 1] = v.y; raw[4 * k + 2] = v.z; raw[4 * k + 3] = v.w;
            }
            const uint8_t* q = p + 16 * W4;
            if constexpr (R == 3) {
                const u32x3_a4 v = ld<NTL>(reinterpret_cast<const u32x3_a4*>(q));
                raw[4 * W4] = v.x; raw[4 * W4 + 1] = v.y; raw[4 * W4 + 2] = v.z;
            } else if constexpr (R == 2) {
                const u32x2_a4 v = ld<NTL>(reinterpret_cast<const u32x2_a4*>(q));
                raw[4 * W4] = v.x; raw[4 * W4 + 1] = v.y;
            } else if constexpr (R == 1) {
                raw[4 * W4] = ld<NTL>(reinterpret_cast<const uint32_t*>(q));
            }
        }
    }
    // The same loads as raw buffer loads on a resource whose base is the wave-uniform `base` of
    // load(), carrying the cache policy bits POL.
    template <int POL>
    static __device__ __forceinline__ void load_buf(__amdgpu_buffer_rsrc_t r, uint32_t ci, uint32_t* raw) {
        const int p = int(ci * K::IB);
        if constexpr (ALIGNED && K::LG == 16) {
#pragma unroll
            for (uint32_t k = 0; k < N / 4; ++k) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, p + 16 * int(k), 0, POL);
                raw[4 * k] = v[0]; raw[4 * k + 1] = v[1]; raw[4 * k + 2] = v[2]; raw[4 * k + 3] = v[3];
            }
        } else if constexpr (ALIGNED && K::LG == 8) {
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, p, 0, POL);
            raw[0] = v[0]; raw[1] = v[1];
        } else if constexpr (ALIGNED) {
            raw[0] = __builtin_amdgcn_raw_buffer_load_b32(r, p, 0, POL);
        } else {
            constexpr uint32_t W4 = RW / 4, R = RW - 4 * W4;
#pragma unroll
            for (uint32_t k = 0; k < W4; ++k) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, p + 16 * int(k), 0, POL);
                raw[4 * k] = v[0]; raw[4 * k + 1] = v[1]; raw[4 * k + 2] = v[2]; raw[4 * k + 3] = v[3];
            }
            const int q = p + 16 * int(W4);
            if constexpr (R == 3) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b96(r, q, 0, POL);
                raw[4 * W4] = v[0]; raw[4 * W4 + 1] = v[1]; raw[4 * W4 + 2] = v[2];
            } else if constexpr (R == 2) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, q, 0, POL);
                raw[4 * W4] = v[0]; raw[4 * W4 + 1] = v[1];
            } else if constexpr (R == 1) {
                raw[4 * W4] = __builtin_amdgcn_raw_buffer_load_b32(r, q, 0, POL);
            }
        }
    }
    static __device__ __forceinline__ void align(const uint32_t* raw, uint32_t sh, uint32_t* in) {
#pragma unroll
        for (uint32_t k = 0; k < N; ++k) in[k] = ALIGNED ? raw[k] : __builtin_amdgcn_alignbyte(raw[k + 1], raw[k], sh);
    }
};

// The scale word of a chunk decoded in the loop (not EARLY_SC), issued ahead of the decode.
template <class K>
__device__ __forceinline__ uint32_t late_sc(const Ctx& c, uint64_t e, uint64_t xs) {
    if constexpr (!K::SC_LOAD) return 0;
    const uint32_t s = K::sc(c, e, xs);
    __builtin_amdgcn_sched_barrier(0);
    return s;
}

// Scale codes of a whole unit of packed fp4 (unit_full, unit_full_paired).  A unit's codes are
// contiguous, one byte per 16 (NVFP4) or 32 (MXFP4) elements: 128 or 64 bytes for the 2048 elements
// of a unit into 2-byte outputs, half that into fp32.  Lane l fetches word l mod W of them (W: the
// unit's 4-byte words of codes), as the 8 bytes from the 4-byte boundary at or below it, issued
// ahead of the data loads; word() realigns it behind the scheduling barrier and code_at hands each
// chunk its code from the lane that holds it (ds_bpermute: every lane of the wavefront is active in
// both unit forms).  Up to 4 bytes past the unit's codes are read, within the blob's tail padding;
// their values are not used.
template <class K>
struct UnitCodes {
    static constexpr uint32_t W = K::UNIT_SB ? K::CE * K::CH * stk::kWave / K::UNIT_SB / 4 : 1;
    u32x2_a4 raw;
    uint32_t sh;
    __device__ __forceinline__ void load(const Ctx& c, uint64_t e0, uint32_t lane) {
        const uint8_t* p = c.blob + c.D.scale + e0 / K::UNIT_SB;
        sh = uint32_t(reinterpret_cast<uintptr_t>(p)) & 3u;
        raw = *reinterpret_cast<const u32x2_a4*>(p - sh + 4 * (lane % W));
    }
    __device__ __forceinline__ uint32_t word() const { return __builtin_amdgcn_alignbyte(raw.y, raw.x, sh); }
};
// Code b of the unit, from the lane whose word holds it
__device__ __forceinline__ uint32_t code_at(uint32_t word, uint32_t b) {
    const uint32_t w = uint32_t(__builtin_amdgcn_ds_bpermute(int((b >> 2) * 4), int(word)));
    return (w >> (8 * (b & 3))) & 0xFFu;
}
// The code of chunk j * 64 + lane of unit_full
template <class K>
__device__ __forceinline__ uint32_t unit_code(uint32_t word, uint32_t j, uint32_t lane) {
    return code_at(word, (j * stk::kWave + lane) * K::CE / K::UNIT_SB);
}
// s_waitcnt vmcnt(0), leaving expcnt and lgkmcnt at their maxima (gfx9 encoding)
constexpr int kWaitVmem0 = 0x0F70;

// The output pointer and the kind's scalar scale, loaded after the unit's data loads are issued.
// False: the output address is not aligned to the output type, and nothing is written.
template <class K, class O>
__device__ __forceinline__ bool finish_ctx(Ctx& c, uint8_t*& out) {
    out = ld_uniform<uint8_t*>(c.outs + c.D.out);
    if constexpr (K::SCALE == 1) c.s = ld_scalar_f32(c.blob + c.D.scale);
    else if constexpr (K::SCALE == 2) c.s = ld_scalar_f32(c.blob + c.D.scale2);
    else c.s = 0.0f;
    const uintptr_t oa = reinterpret_cast<uintptr_t>(out);
    c.vec = (oa & 15u) == 0;
    return (oa & (O::BYTES - 1)) == 0;
}

// Exact path for the n elements from e, one at a time.  Kept as a loop (not unrolled): this is
// the cold path, and unrolled copies of it at every call site made the kernel's code several
// times larger, which was measured to cost 1-3% of bandwidth on the fast path.
template <uint32_t KIND, class O>
__device__ __forceinline__ void run_exact(const Ctx& c, uint8_t* __restrict__ out, uint64_t e, uint32_t n) {
#pragma unroll 1
    for (uint32_t k = 0; k < n; ++k) store_elem<O>(out, e + k, kind_exact<KIND, O>(c.blob, c.D, e + k));
}

// One 16-byte output word at byte offset off from the wave-uniform address base.  NT: the table's
// outputs exceed the last-level cache, so they are streamed past it rather than kept there (smaller
// tables' outputs stay in that cache for whatever reads them next).  The streaming store is a raw
// buffer store with the non-temporal bit and system scope (nt sc1): measured against the
// non-temporal bit alone, +0.3 to +1.6%; system scope alone, or with sc0, was slower.  A global store
// cannot carry sc1 from HIP, hence the buffer resource built on base, which must be uniform.
constexpr int kRawBufferWord3 = 0x00020000;  // V# word 3 of an untyped buffer (32-bit data format)
constexpr int kStreamStorePolicy = 2 | 16;   // cache policy bits: nt | sc1
// Data loads of whole units in the streaming-store instances: non-temporal (nt) for bf16 copies and
// MXFP8, the default policy for the other kinds.  Measured on MI355X against the default policy, in
// one process: block-FP8 checkpoint with its bf16 embedding +1.1% (the embedding's share), MXFP8 +3.5%;
// scaled FP8 -1.7%, NVFP4 -1.3% (unchanged when left out), block FP8 alone and MXFP4 unchanged.  The
// plain-store instances (outputs that fit the last-level cache) keep the default policy: non-temporal
// loads there cost the many-small checkpoint 11% after a clean cache flush.
constexpr int kStreamLoadPolicy = 2;  // nt
// Whole units of column slices (a strided source, one descriptor per slice) of the fp4, MXFP8 and
// scaled-FP8 kinds load non-temporally.  Measured on MI355X against default loads, one rank's column
// shard of every 2-d weight of the large checkpoints (same process): NVFP4 +3.7%, MXFP4 +8.6%, MXFP8
// +13%, scaled FP8 +0.9%; the block-FP8 checkpoint's 8-way column shards lost 1.1%, so block FP8
// (and the 2- and 4-byte sources, not measured) keep the default.  Split descriptors, which read
// whole rows, lost 2-4% with non-temporal loads and keep the default too.
template <class K>
constexpr bool slice_loads_nt() {
    return K::KIND == ST_KIND_NVFP4 || K::KIND == ST_KIND_MXFP4 || K::KIND == ST_KIND_MXFP8 ||
           K::KIND == ST_KIND_FP8_TENSOR;
}
template <class K, class O>
constexpr int load_policy() {
    return O::NT && (K::KIND == ST_KIND_PASS_BF16 || K::KIND == ST_KIND_MXFP8) ? kStreamLoadPolicy : 0;
}
template <bool NT>
__device__ __forceinline__ void store_word(uint8_t* base, uint32_t off, u32x4 v) {
    if constexpr (NT) {
        const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(base, 0, 0x7FFFFFFF, kRawBufferWord3);
        __builtin_amdgcn_raw_buffer_store_b128(v, r, int(off), 0, kStreamStorePolicy);
    } else {
        *reinterpret_cast<u32x4*>(base + off) = v;
    }
}

// The output words of chunk ci of a unit whose output starts at ob, as 16-byte stores.  ob is
// wave-uniform and the chunk's offset a 32-bit lane value, so the stores take a scalar base and a
// 32-bit vector offset (a 64-bit address per lane costs measurably more store bandwidth).
template <class K, class O>
__device__ __forceinline__ void store_chunk(uint8_t* __restrict__ ob, uint32_t ci, const uint32_t* w) {
    constexpr uint32_t OW = K::CE * O::BYTES / 16;
    const uint32_t off = ci * (K::CE * O::BYTES);
#pragma unroll
    for (uint32_t k = 0; k < OW; ++k)
        store_word<O::NT>(ob, off + 16 * k, u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]});
}

// A unit of exactly CH * 64 whole chunks (the default unit size): no per-chunk bounds checks.
template <class K, class O, bool ALIGNED>
__device__ __forceinline__ void unit_full(const Ctx& c0, uint64_t e0, uint32_t sh, uint32_t lane) {
    using F = Fetch<K, ALIGNED>;
    constexpr uint32_t NW = K::CE * O::BYTES / 4;
    const uint8_t* base = c0.blob + c0.D.src + K::src_off(e0) - sh;
    uint32_t raw[K::CH][F::RW], sc[K::CH];
    UnitCodes<K> codes;
    if constexpr (K::UNIT_SB != 0) codes.load(c0, e0, lane);
    if constexpr (load_policy<K, O>() != 0) {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, 0x7FFFFFFF, kRawBufferWord3);
#pragma unroll
        for (uint32_t j = 0; j < K::CH; ++j) F::template load_buf<load_policy<K, O>()>(r, j * stk::kWave + lane, raw[j]);
    } else {
#pragma unroll
        for (uint32_t j = 0; j < K::CH; ++j) F::load(base, j * stk::kWave + lane, raw[j]);
    }
    if constexpr (K::EARLY_SC) {
#pragma unroll
        for (uint32_t j = 0; j < K::CH; ++j) {
            const uint64_t e = e0 + uint64_t(j * stk::kWave + lane) * K::CE;
            sc[j] = K::sc(c0, e, e);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    Ctx c = c0;
    uint8_t* out;
    // The data loads go out first.  The scheduling barrier keeps the output pointer's and the
    // scale's scalar loads (and their wait) behind them, and no branch on those values precedes
    // the decode: the output check and the fast-path conditions are combined with & afterwards,
    // so the compiler cannot sink the data loads behind a round trip.  Measured on MI355X: +1% on
    // scaled FP8, +3.5% on NVFP4, +8.5% on MXFP8, +4.5% on many small tensors.
    const bool valid = finish_ctx<K, O>(c, out);
    const bool vec = valid & c.vec;
    uint8_t* const ob = out + e0 * O::BYTES;
    uint32_t code_word = 0;
    if constexpr (K::UNIT_SB != 0) code_word = codes.word();
    bool ok[K::CH];
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j) {
        const uint64_t e = e0 + uint64_t(j * stk::kWave + lane) * K::CE;
        uint32_t s;
        if constexpr (K::UNIT_SB != 0) s = unit_code<K>(code_word, j, lane);
        else s = K::EARLY_SC ? sc[j] : late_sc<K>(c, e, e);
        uint32_t in[F::N], w[NW];
        F::align(raw[j], sh, in);
        ok[j] = K::fast(c, in, s, w) & vec;
        if (ok[j]) store_chunk<K, O>(ob, j * stk::kWave + lane, w);
        // Packed fp4: each chunk's store completes before the next chunk's is issued.  Measured on
        // MI355X, NVFP4 / MXFP4 checkpoints: with this wait the unit-wide code fetch gains 1.0% /
        // 0.7% over per-chunk code loads (whose own waits spaced the stores the same way); without
        // it, it loses 2-3%.  Waits that leave one or two stores in flight, or a single wait after
        // the second chunk, lost 0.8-2%; the same wait on the 8-bit and 2-byte kinds lost 1-2%.
        if constexpr (K::UNIT_SB != 0) {
            if (j + 1 < K::CH) __builtin_amdgcn_s_waitcnt(kWaitVmem0);
        }
    }
    bool all = true;
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j) all &= ok[j];
    if (__builtin_amdgcn_ballot_w64(!all) == 0 || !valid) return;  // the common case; or no output
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j)
        if (!ok[j]) run_exact<K::KIND, O>(c, out, e0 + uint64_t(j * stk::kWave + lane) * K::CE, K::CE);
}

// A whole unit of packed fp4 into fp32.  A lane's 4-byte load holds 8 elements, 32 bytes of
// output; stored as two adjacent 16-byte words per lane, every store instruction of the wave would
// leave a 16-byte gap after each lane's word.  Instead, for the 512 elements of load step j, lanes
// 2i and 2i + 1 load the words of chunks i and 32 + i and swap 16-bit halves with a DPP quad
// permutation, so that lane l holds elements 4l..4l+3 and 256+4l..256+4l+3: each of the two store
// instructions then covers 1024 contiguous bytes.  The same chunks are loaded as in unit_full.
template <class K, class O, bool ALIGNED>
__device__ __forceinline__ void unit_full_paired(const Ctx& c0, uint64_t e0, uint32_t sh, uint32_t lane) {
    using F = Fetch<K, ALIGNED>;
    static_assert(K::CE == 8 && F::N == 1 && O::BYTES == 4, "8 packed fp4 elements per 4-byte word");
    constexpr uint32_t GE = K::CE * stk::kWave;  // elements per load step
    const uint8_t* base = c0.blob + c0.D.src + K::src_off(e0) - sh;
    const bool odd = (lane & 1u) != 0;
    const uint32_t mine = (lane >> 1) + (odd ? stk::kWave / 2 : 0u);  // the chunk this lane loads
    uint32_t raw[K::CH][F::RW];
    // The unit's scale codes as in unit_full; here without waits between the stores.  Measured on
    // MI355X into fp32 against per-chunk code loads: NVFP4 +1.3%, MXFP4 +2.8% (same process); with
    // the waits, no change.
    UnitCodes<K> codes;
    codes.load(c0, e0, lane);
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j) F::load(base, j * stk::kWave + mine, raw[j]);
    __builtin_amdgcn_sched_barrier(0);
    Ctx c = c0;
    uint8_t* out;
    const bool valid = finish_ctx<K, O>(c, out);  // as in unit_full: no branch before the decode
    const bool vec = valid & c.vec;
    uint8_t* const ob = out + e0 * O::BYTES;
    const uint32_t code_word = codes.word();
    bool ok[K::CH];
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j) {
        const uint64_t ea = e0 + j * GE + 4 * lane, eb = ea + GE / 2;
        const uint32_t sa = code_at(code_word, (j * GE + 4 * lane) / K::UNIT_SB),
                       sb = code_at(code_word, (j * GE + GE / 2 + 4 * lane) / K::UNIT_SB);
        uint32_t in[1];
        F::align(raw[j], sh, in);
        // quad_perm(1, 0, 3, 2): the value of lane l ^ 1
        const uint32_t mate = uint32_t(__builtin_amdgcn_mov_dpp(int(in[0]), 0xB1, 0xF, 0xF, false));
        // even lane: its own low half, then its mate's; odd lane: its mate's high half, then its own
        const uint32_t x = odd ? __builtin_amdgcn_perm(in[0], mate, 0x07060302u)
                               : __builtin_amdgcn_perm(mate, in[0], 0x05040100u);
        uint32_t wa[4], wb[4];
        ok[j] = K::template quad<0>(c, x, sa, wa) & K::template quad<2>(c, x, sb, wb) & vec;
        if (ok[j]) {
            const uint32_t off = (j * GE + 4 * lane) * O::BYTES;
            store_word<O::NT>(ob, off, u32x4{wa[0], wa[1], wa[2], wa[3]});
            store_word<O::NT>(ob, off + GE / 2 * O::BYTES, u32x4{wb[0], wb[1], wb[2], wb[3]});
        }
    }
    bool all = true;
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j) all &= ok[j];
    if (__builtin_amdgcn_ballot_w64(!all) == 0 || !valid) return;
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j)
        if (!ok[j]) {
            const uint64_t ea = e0 + j * GE + 4 * lane;
            run_exact<K::KIND, O>(c, out, ea, 4);
            run_exact<K::KIND, O>(c, out, ea + GE / 2, 4);
        }
}

// Any unit: cnt elements (a larger unit size, or an output's final unit).
template <class K, class O, bool ALIGNED>
__device__ __forceinline__ void unit_any(const Ctx& c0, uint64_t e0, uint32_t cnt, uint32_t sh, uint32_t lane) {
    using F = Fetch<K, ALIGNED>;
    constexpr uint32_t NW = K::CE * O::BYTES / 4;
    Ctx c = c0;
    uint8_t* out;
    if (!finish_ctx<K, O>(c, out)) return;
    const uint8_t* base = c.blob + c.D.src + K::src_off(e0) - sh;
    uint8_t* const ob = out + e0 * O::BYTES;
    const uint32_t nch = cnt / K::CE;  // whole chunks
    for (uint32_t ci = lane; ci < nch; ci += stk::kWave) {
        uint32_t raw[F::RW], in[F::N], w[NW];
        F::load(base, ci, raw);
        F::align(raw, sh, in);
        const uint64_t e = e0 + uint64_t(ci) * K::CE;
        if (c.vec && K::fast(c, in, K::sc(c, e, e), w)) store_chunk<K, O>(ob, ci, w);
        else run_exact<K::KIND, O>(c, out, e, K::CE);
    }
#pragma unroll 1
    for (uint32_t t = nch * K::CE + lane; t < cnt; t += stk::kWave)  // past the last whole chunk
        store_elem<O>(out, e0 + t, kind_exact<K::KIND, O>(c.blob, c.D, e0 + t));
}

// A whole unit of a column slice: chunk starts are mapped to their source elements one by one
// (the host guarantees that a chunk never crosses a row and that every chunk has the alignment of
// the slice's first source byte, or marks the descriptor exact-only).  All of a lane's loads are
// issued before decoding, like unit_full.
template <class K, class O, bool ALIGNED>
__device__ __forceinline__ void unit_strided_full(const Ctx& c0, uint64_t e0, uint32_t sh, uint32_t lane) {
    using F = Fetch<K, ALIGNED>;
    constexpr uint32_t NW = K::CE * O::BYTES / 4;
    const uint8_t* base = c0.blob + c0.D.src - sh;
    uint32_t raw[K::CH][F::RW], sc[K::CH];
    uint64_t xs[K::CH];
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j) {
        const uint64_t e = e0 + uint64_t(j * stk::kWave + lane) * K::CE;
        xs[j] = src_elem(c0.D, e);
        F::template load<slice_loads_nt<K>()>(base + K::src_off(xs[j]), 0, raw[j]);
        if constexpr (K::EARLY_SC) sc[j] = K::sc(c0, e, xs[j]);
    }
    __builtin_amdgcn_sched_barrier(0);
    Ctx c = c0;
    uint8_t* out;
    const bool valid = finish_ctx<K, O>(c, out);  // combined after decoding, as in unit_full
    const bool vec = valid & c.vec;
    uint8_t* const ob = out + e0 * O::BYTES;
    bool ok[K::CH];
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j) {
        const uint64_t e = e0 + uint64_t(j * stk::kWave + lane) * K::CE;
        const uint32_t s = K::EARLY_SC ? sc[j] : late_sc<K>(c, e, xs[j]);
        uint32_t in[F::N], w[NW];
        F::align(raw[j], sh, in);
        ok[j] = K::fast(c, in, s, w) & vec;
        if (ok[j]) store_chunk<K, O>(ob, j * stk::kWave + lane, w);
    }
    bool all = true;
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j) all &= ok[j];
    if (__builtin_amdgcn_ballot_w64(!all) == 0 || !valid) return;
#pragma unroll
    for (uint32_t j = 0; j < K::CH; ++j)
        if (!ok[j]) run_exact<K::KIND, O>(c, out, e0 + uint64_t(j * stk::kWave + lane) * K::CE, K::CE);
}

// A partial unit of a column slice (or any unit of a larger unit size): the lane walks its chunks,
// then the elements past the last whole chunk.  Unaligned loads, correct at any alignment.
template <class K, class O>
__device__ __forceinline__ void unit_strided_any(const Ctx& c0, uint64_t e0, uint32_t cnt, uint32_t sh, uint32_t lane) {
    using F = Fetch<K, false>;
    constexpr uint32_t NW = K::CE * O::BYTES / 4;
    const uint8_t* base = c0.blob + c0.D.src - sh;
    Ctx c = c0;
    uint8_t* out;
    if (!finish_ctx<K, O>(c, out)) return;
    uint8_t* const ob = out + e0 * O::BYTES;
    const uint32_t nch = cnt / K::CE;
    for (uint32_t ci = lane; ci < nch; ci += stk::kWave) {
        const uint64_t e = e0 + uint64_t(ci) * K::CE;
        const uint64_t x = src_elem(c.D, e);
        uint32_t raw[F::RW], in[F::N], w[NW];
        F::load(base + K::src_off(x), 0, raw);
        F::align(raw, sh, in);
        if (c.vec && K::fast(c, in, K::sc(c, e, x), w)) store_chunk<K, O>(ob, ci, w);
        else run_exact<K::KIND, O>(c, out, e, K::CE);
    }
#pragma unroll 1
    for (uint32_t t = nch * K::CE + lane; t < cnt; t += stk::kWave)
        store_elem<O>(out, e0 + t, kind_exact<K::KIND, O>(c.blob, c.D, e0 + t));
}

template <class K, class O>
__device__ __forceinline__ void run_strided(const Ctx& c, uint64_t e0, uint32_t cnt, uint32_t lane) {
    const uint32_t a = uint32_t(reinterpret_cast<uintptr_t>(c.blob + c.D.src));
    if (cnt != K::CE * K::CH * stk::kWave) unit_strided_any<K, O>(c, e0, cnt, a & 3u, lane);
    else if ((a & (K::LG - 1)) == 0) unit_strided_full<K, O, true>(c, e0, 0, lane);
    else unit_strided_full<K, O, false>(c, e0, a & 3u, lane);
}

// Every element of a unit through the exact path (descriptors the host marks exact-only).
template <uint32_t KIND, class O>
__device__ __forceinline__ void unit_exact(const Ctx& c, uint64_t e0, uint32_t cnt, uint32_t lane) {
    if (c.D.flags & ST_DESC_SPLIT) {  // each element to its shard
        if constexpr (KIND == ST_KIND_FP8_BLOCK128) return;  // never planned: its scale grid needs cols
#pragma unroll 1
        for (uint32_t t = lane; t < cnt; t += stk::kWave) {
            uint32_t s;
            const uint32_t i = split_dst(c.D, e0 + t, &s);
            uint8_t* out = c.outs[c.D.out + s];
            if ((reinterpret_cast<uintptr_t>(out) & (O::BYTES - 1)) == 0)
                store_elem<O>(out, i, kind_exact<KIND, O>(c.blob, c.D, e0 + t));
        }
        return;
    }
    uint8_t* out = ld_uniform<uint8_t*>(c.outs + c.D.out);
    if (reinterpret_cast<uintptr_t>(out) & (O::BYTES - 1)) return;
#pragma unroll 1
    for (uint32_t t = lane; t < cnt; t += stk::kWave) store_elem<O>(out, e0 + t, kind_exact<KIND, O>(c.blob, c.D, e0 + t));
}

// Stores one chunk of a split descriptor to its shard (p: the chunk's output address); chunks the fast
// path cannot take (NaN inputs, non-finite scales, a shard not 16-byte aligned) go element by element.
template <class K, class O>
__device__ __forceinline__ void split_store(const Ctx& c, const uint32_t* in, uint32_t s, uint8_t* shard,
                                            uint32_t idx, uint64_t e) {
    constexpr uint32_t NW = K::CE * O::BYTES / 4;
    uint32_t w[NW];
    uint8_t* p = shard + size_t(idx) * O::BYTES;
    if ((reinterpret_cast<uintptr_t>(p) & 15u) == 0 && K::fast(c, in, s, w)) {
        // A pointer taken from another lane is generic to the compiler: without the global address
        // space the stores are flat ones, which also count against the LDS/scalar wait counter, so
        // every later wait for a cross-lane read or a scalar load would wait for them.
        global_u32x4* g = (global_u32x4*)(p);
#pragma unroll
        for (uint32_t k = 0; k < NW / 4; ++k) g[k] = u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
    } else if ((reinterpret_cast<uintptr_t>(shard) & (O::BYTES - 1)) == 0) {
#pragma unroll 1
        for (uint32_t k = 0; k < K::CE; ++k) store_elem<O>(shard, idx + k, kind_exact<K::KIND, O>(c.blob, c.D, e + k));
    }
}

// A whole unit of a split descriptor (every column shard of some rows in one descriptor; see
// split_dst): the source is read whole, like a whole output, with the same load order as unit_full,
// and each chunk is stored to its shard.  A chunk never crosses a shard (cols is a whole number of
// chunks), so it is still one 16-byte output word, at a per-lane address; its offset in the shard is
// a multiple of 16 bytes, so the shards' own alignment decides the vector stores, once per unit.
// Lane l loads shard (l mod 2^grid_cols)'s output pointer once; each chunk takes its shard's from
// that lane.  Every lane of the wave is active here (the unit test is wave-uniform), as that
// cross-lane read needs.  As in unit_full, chunks the fast path cannot take go element by element
// after all the fast stores.
template <class K, class O, bool ALIGNED>
__device__ __forceinline__ void unit_split_full(const Ctx& c0, uint64_t e0, uint32_t sh, uint32_t lane) {
    using F = Fetch<K, ALIGNED>;
    constexpr uint32_t NW = K::CE * O::BYTES / 4, CH = K::CH;
    const uint8_t* base = c0.blob + c0.D.src + K::src_off(e0) - sh;
    uint32_t raw[CH][F::RW];
#pragma unroll
    for (uint32_t j = 0; j < CH; ++j) F::load(base, j * stk::kWave + lane, raw[j]);
    const uint64_t mine =
        reinterpret_cast<uint64_t>(c0.outs[c0.D.out + (lane & ((1u << c0.D.grid_cols) - 1u))]);
    __builtin_amdgcn_sched_barrier(0);
    Ctx c = c0;
    uint8_t* first;
    (void)finish_ctx<K, O>(c, first);  // the scalar scale; the shards' pointers are checked below
    bool ok[CH], vec = false;
#pragma unroll
    for (uint32_t j = 0; j < CH; ++j) {
        const uint64_t e = e0 + uint64_t(j * stk::kWave + lane) * K::CE;
        const uint32_t s = late_sc<K>(c, e, e);
        // every shard 16-byte aligned; taken after the first scale load is issued, so that one wait
        // covers the data, the pointers and that scale, as in unit_full
        if (j == 0) vec = __builtin_amdgcn_ballot_w64((mine & 15u) != 0) == 0;
        uint32_t which, in[F::N], w[NW];
        const uint32_t idx = split_dst(c.D, e, &which);
        const int from = int(which << 2);
        const uint32_t lo = uint32_t(__builtin_amdgcn_ds_bpermute(from, int(uint32_t(mine))));
        const uint32_t hi = uint32_t(__builtin_amdgcn_ds_bpermute(from, int(uint32_t(mine >> 32))));
        F::align(raw[j], sh, in);
        ok[j] = K::fast(c, in, s, w) & vec;
        if (ok[j]) {
            global_u32x4* g = (global_u32x4*)(reinterpret_cast<uint8_t*>(uint64_t(hi) << 32 | lo) + size_t(idx) * O::BYTES);
#pragma unroll
            for (uint32_t k = 0; k < NW / 4; ++k) g[k] = u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
        }
    }
    bool all = true;
#pragma unroll
    for (uint32_t j = 0; j < CH; ++j) all &= ok[j];
    if (__builtin_amdgcn_ballot_w64(!all) == 0) return;  // the common case
#pragma unroll
    for (uint32_t j = 0; j < CH; ++j) {
        if (ok[j]) continue;
        const uint64_t e = e0 + uint64_t(j * stk::kWave + lane) * K::CE;
        uint32_t which;
        const uint32_t idx = split_dst(c.D, e, &which);
        uint8_t* shard = c.outs[c.D.out + which];
        if ((reinterpret_cast<uintptr_t>(shard) & (O::BYTES - 1)) != 0) continue;
#pragma unroll 1
        for (uint32_t k = 0; k < K::CE; ++k) store_elem<O>(shard, idx + k, kind_exact<K::KIND, O>(c.blob, c.D, e + k));
    }
}

// A partial unit of a split descriptor (its last, or any unit of a larger unit size): the lane walks
// its chunks with unaligned loads, correct at any alignment, each loading its shard's pointer.
template <class K, class O>
__device__ __forceinline__ void unit_split_any(const Ctx& c0, uint64_t e0, uint32_t cnt, uint32_t sh, uint32_t lane) {
    using F = Fetch<K, false>;
    const uint8_t* base = c0.blob + c0.D.src + K::src_off(e0) - sh;
    Ctx c = c0;
    uint8_t* first;
    (void)finish_ctx<K, O>(c, first);
    const uint32_t nch = cnt / K::CE;
    for (uint32_t ci = lane; ci < nch; ci += stk::kWave) {
        const uint64_t e = e0 + uint64_t(ci) * K::CE;
        uint32_t raw[F::RW], in[F::N], which;
        F::load(base, ci, raw);
        const uint32_t idx = split_dst(c.D, e, &which);
        F::align(raw, sh, in);
        split_store<K, O>(c, in, K::sc(c, e, e), c.outs[c.D.out + which], idx, e);
    }
}

// A whole unit takes the aligned or unaligned fast path by its source alignment; a partial unit (an
// output's last, or any unit of a larger unit size) always takes the unaligned form, which is
// correct at any alignment, so that the kernel holds one copy of it per kind.  Aligned: the source
// starts on an LG-byte boundary; otherwise sh = its offset within a 4-byte word (0 for a
// 4-byte-aligned source that is not LG-aligned).
template <class K, class O>
__device__ __forceinline__ void run_unit(const Ctx& c, uint64_t e0, uint32_t cnt, uint32_t lane) {
    const uint32_t a = uint32_t(reinterpret_cast<uintptr_t>(c.blob + c.D.src + K::src_off(e0)));
    if (cnt != K::CE * K::CH * stk::kWave) unit_any<K, O, false>(c, e0, cnt, a & 3u, lane);
    else if constexpr (K::PAIRED) {
        if ((a & (K::LG - 1)) == 0) unit_full_paired<K, O, true>(c, e0, 0, lane);
        else unit_full_paired<K, O, false>(c, e0, a & 3u, lane);
    } else if ((a & (K::LG - 1)) == 0) unit_full<K, O, true>(c, e0, 0, lane);
    else unit_full<K, O, false>(c, e0, a & 3u, lane);
}

// ------------------------------------------------------------------------- the kernel

// The split kinds as a bit mask (bit k set when stk::split_kind(k)): the kernel tests a descriptor's
// kind against it instead of calling the shared predicate, which the compiler left out of line in
// the large kernels.
constexpr uint32_t split_kind_mask() {
    uint32_t m = 0;
    for (uint32_t k = 0; k < 32; ++k) m |= uint32_t(stk::split_kind(k)) << k;
    return m;
}
constexpr uint32_t kSplitKinds = split_kind_mask();

// SLICES: the instance that runs column slices through the strided fast path.  The plain instance
// sends them (and exact-only descriptors) through the per-element exact path; keeping the strided
// code out of it was measured to matter (2-5% on the whole-checkpoint decode).  O: the output
// type; a table planned for another output type is left alone.
template <bool SLICES, class O>
__global__ __launch_bounds__(kBlock) void materialize_kernel(const uint8_t* __restrict__ blob,
                                                             const uint8_t* __restrict__ table, uint32_t units,
                                                             uint32_t groups, uint32_t desc_off,
                                                             uint8_t* const* __restrict__ outs) {
    // XCD-contiguous renumbering: workgroup b runs on XCD b % 8; XCD x gets the contiguous range
    // of groups [start_x, start_x + count_x), a bijection of [0, groups).
    const uint32_t b = blockIdx.y * gridDim.x + blockIdx.x;
    if (b >= groups) return;
    const uint32_t x = b & 7u, q = groups >> 3, rem = groups & 7u;
    const uint32_t grp = x * q + (x < rem ? x : rem) + (b >> 3);
    const uint32_t unit = grp * ST_UNITS_PER_GROUP + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (unit >= units) return;
    const uint32_t lane = threadIdx.x & (stk::kWave - 1);

    // Header (magic, unit count, output type), this group's map entry, then the descriptor: the
    // only loads ahead of the data.  A table that does not match n or this instance's output type
    // is left alone before anything indexes it.
    const u32x4 hw = ld_uniform<u32x4>(table);
    const uint32_t odt = ld_uniform<uint32_t>(table + offsetof(st_table_header, out_dtype));
    if ((hw.x != ST_TABLE_MAGIC) | (hw.z != units) | (hw.w != 0) | (odt != O::CODE)) return;
    uint32_t d = ld_uniform<uint32_t>(table + sizeof(st_table_header) + 4 * size_t(grp));
    const st_desc* descs = reinterpret_cast<const st_desc*>(table + desc_off);
    Desc D = load_desc(descs + d);
    while (unit >= D.unit_end) D = load_desc(descs + (++d));  // up to 3 steps, plus empty outputs

    const uint64_t e0 = uint64_t(unit - D.unit_begin) << D.unit_shift;
    const uint32_t cnt = unit + 1 == D.unit_end ? D.tail : 1u << D.unit_shift;
    Ctx c;
    c.blob = blob;
    c.D = D;
    c.outs = outs;
    c.scale_al = (D.scale & 3u) == 0;
    if ((D.pitch | D.flags) != 0) {  // column slices, split descriptors and exact-only descriptors
        if (SLICES && (D.flags & (ST_DESC_SPLIT | ST_DESC_EXACT)) == ST_DESC_SPLIT && (cnt & 7u) == 0 &&
            D.kind < 32u && ((kSplitKinds >> D.kind) & 1u)) {
            const uint32_t a = uint32_t(reinterpret_cast<uintptr_t>(c.blob + c.D.src)), sh = a & 3u;
            switch (D.kind) {
            // whole units of the default size take the unrolled form, the others walk their chunks
#define ST_SPLIT_CASE(KIND_, K_)                                                                  \
    case KIND_:                                                                                   \
        static_assert(stk::split_kind(KIND_), "a split kind");                                    \
        {                                                                                         \
            const bool full_ = cnt == (1u << D.unit_shift) && D.unit_shift == stk::step_shift(KIND_, O::CODE); \
            const bool al_ = (a & (K_<O>::LG - 1)) == 0;                                          \
            if (full_) al_ ? unit_split_full<K_<O>, O, true>(c, e0, 0, lane)                      \
                           : unit_split_full<K_<O>, O, false>(c, e0, sh, lane);                   \
            else unit_split_any<K_<O>, O>(c, e0, cnt, sh, lane);                                  \
        }                                                                                         \
        break;
                ST_SPLIT_CASE(ST_KIND_NVFP4, KFp4)
                ST_SPLIT_CASE(ST_KIND_MXFP4, KMx4)
#undef ST_SPLIT_CASE
                default: break;  // not a split kind
            }
            return;
        }
        if (!SLICES || (D.flags & (ST_DESC_EXACT | ST_DESC_SPLIT))) {
            switch (D.kind) {
                case ST_KIND_FP8_TENSOR: unit_exact<ST_KIND_FP8_TENSOR, O>(c, e0, cnt, lane); break;
                case ST_KIND_FP8_BLOCK128: unit_exact<ST_KIND_FP8_BLOCK128, O>(c, e0, cnt, lane); break;
                case ST_KIND_NVFP4: unit_exact<ST_KIND_NVFP4, O>(c, e0, cnt, lane); break;
                case ST_KIND_PASS_BF16: unit_exact<ST_KIND_PASS_BF16, O>(c, e0, cnt, lane); break;
                case ST_KIND_CAST_F16: unit_exact<ST_KIND_CAST_F16, O>(c, e0, cnt, lane); break;
                case ST_KIND_MXFP8: unit_exact<ST_KIND_MXFP8, O>(c, e0, cnt, lane); break;
                case ST_KIND_MXFP4: unit_exact<ST_KIND_MXFP4, O>(c, e0, cnt, lane); break;
                default: unit_exact<ST_KIND_CAST_F32, O>(c, e0, cnt, lane); break;
            }
            return;
        }
        switch (D.kind) {
            case ST_KIND_FP8_TENSOR: run_strided<KFp8Tensor<O>, O>(c, e0, cnt, lane); break;
            case ST_KIND_FP8_BLOCK128: run_strided<KFp8Block<O>, O>(c, e0, cnt, lane); break;
            case ST_KIND_NVFP4: run_strided<KFp4<O>, O>(c, e0, cnt, lane); break;
            case ST_KIND_PASS_BF16: run_strided<KPass<O>, O>(c, e0, cnt, lane); break;
            case ST_KIND_CAST_F16: run_strided<KF16<O>, O>(c, e0, cnt, lane); break;
            case ST_KIND_MXFP8: run_strided<KMx8<O>, O>(c, e0, cnt, lane); break;
            case ST_KIND_MXFP4: run_strided<KMx4<O>, O>(c, e0, cnt, lane); break;
            default: run_strided<KF32<O>, O>(c, e0, cnt, lane); break;
        }
        return;
    }
    switch (D.kind) {
        case ST_KIND_FP8_TENSOR: run_unit<KFp8Tensor<O>, O>(c, e0, cnt, lane); break;
        case ST_KIND_FP8_BLOCK128: run_unit<KFp8Block<O>, O>(c, e0, cnt, lane); break;
        case ST_KIND_NVFP4: run_unit<KFp4<O>, O>(c, e0, cnt, lane); break;
        case ST_KIND_PASS_BF16: run_unit<KPass<O>, O>(c, e0, cnt, lane); break;
        case ST_KIND_CAST_F16: run_unit<KF16<O>, O>(c, e0, cnt, lane); break;
        case ST_KIND_MXFP8: run_unit<KMx8<O>, O>(c, e0, cnt, lane); break;
        case ST_KIND_MXFP4: run_unit<KMx4<O>, O>(c, e0, cnt, lane); break;
        default: run_unit<KF32<O>, O>(c, e0, cnt, lane); break;
    }
}

template <bool SLICES, class O, bool NT>
void launch_as(const void* blob, const void* descs, uint32_t n, uint32_t groups, void* const* outs, hipStream_t stream) {
    const uint32_t gx = groups < kMaxGridX ? groups : kMaxGridX;
    const uint32_t gy = (groups + gx - 1) / gx;
    hipLaunchKernelGGL((materialize_kernel<SLICES, Stored<O, NT>>), dim3(gx, gy), dim3(kBlock), 0, stream,
                       static_cast<const uint8_t*>(blob), static_cast<const uint8_t*>(descs), n, groups,
                       uint32_t(stk::table_desc_offset(groups)), reinterpret_cast<uint8_t* const*>(outs));
}

template <bool SLICES, class O>
void launch(const void* blob, const void* descs, uint32_t n, uint32_t groups, void* const* outs, hipStream_t stream,
            bool nt) {
    nt ? launch_as<SLICES, O, true>(blob, descs, n, groups, outs, stream)
       : launch_as<SLICES, O, false>(blob, descs, n, groups, outs, stream);
}

}  // namespace

extern "C" st_status st_materialize_as(const void* blob, const void* descs, size_t n, void* const* outs,
                                       uint32_t out_dtype, uint32_t flags, void* stream) {
    const char* who = "st_materialize";
    if (n == 0) return ST_OK;
    if (!blob || !descs || !outs) return st_fail(ST_E_ARG, "%s: null pointer", who);
    if (reinterpret_cast<uintptr_t>(blob) % ST_BLOB_ALIGN)
        return st_fail(ST_E_ARG, "%s: blob is not %d-byte aligned", who, ST_BLOB_ALIGN);
    if (reinterpret_cast<uintptr_t>(descs) % 64) return st_fail(ST_E_ARG, "%s: work table is not 64-byte aligned", who);
    if (uint64_t(n) >= (uint64_t(1) << 32)) return st_fail(ST_E_ARG, "%s: %zu work units (at most 2^32 - 1)", who, n);
    if (out_dtype > ST_OUT_F32) return st_fail(ST_E_ARG, "%s: unknown output type %u", who, out_dtype);
    if (flags & ~uint32_t(ST_MAT_SLICES | ST_MAT_STREAM_STORES)) return st_fail(ST_E_ARG, "%s: unknown flags 0x%x", who, flags);
    const uint32_t groups = uint32_t((uint64_t(n) + ST_UNITS_PER_GROUP - 1) / ST_UNITS_PER_GROUP);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool slices = (flags & ST_MAT_SLICES) != 0, nt = (flags & ST_MAT_STREAM_STORES) != 0;
    switch (out_dtype) {
        case ST_OUT_BF16:
            slices ? launch<true, OutBf16>(blob, descs, uint32_t(n), groups, outs, s, nt)
                   : launch<false, OutBf16>(blob, descs, uint32_t(n), groups, outs, s, nt);
            break;
        case ST_OUT_F16:
            slices ? launch<true, OutF16>(blob, descs, uint32_t(n), groups, outs, s, nt)
                   : launch<false, OutF16>(blob, descs, uint32_t(n), groups, outs, s, nt);
            break;
        default:
            slices ? launch<true, OutF32>(blob, descs, uint32_t(n), groups, outs, s, nt)
                   : launch<false, OutF32>(blob, descs, uint32_t(n), groups, outs, s, nt);
            break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return st_fail(ST_E_HIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    return ST_OK;
}

namespace {

constexpr int kMaxDevices = 64;

// The address of `scratch` on device `dev`, looked up once per device with that device current.
st_status scratch_address(int dev, uint8_t** out) {
    static std::mutex m;
    static uint8_t* addr[kMaxDevices] = {};
    if (dev < 0 || dev >= kMaxDevices) return st_fail(ST_E_ARG, "st_materialize_noalloc: device %d out of range", dev);
    std::lock_guard<std::mutex> lk(m);
    if (!addr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return st_fail(ST_E_HIP, "st_materialize_noalloc: hipGetDevice failed");
        if (cur != dev && hipSetDevice(dev) != hipSuccess)
            return st_fail(ST_E_HIP, "st_materialize_noalloc: hipSetDevice(%d) failed", dev);
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p)
            return st_fail(ST_E_HIP, "st_materialize_noalloc: hipGetSymbolAddress of the scratch array failed on device %d: %s",
                           dev, hipGetErrorString(e));
        addr[dev] = static_cast<uint8_t*>(p);
    }
    *out = addr[dev];
    return ST_OK;
}

}  // namespace

extern "C" st_status st_materialize_noalloc(const void* blob, const void* table_host, size_t table_bytes, size_t n,
                                            void* const* outs_host, size_t n_outs, uint32_t out_dtype, uint32_t flags,
                                            void* stream) {
    const char* who = "st_materialize_noalloc";
    if (n == 0) return ST_OK;
    if (!blob || !table_host || (n_outs && !outs_host)) return st_fail(ST_E_ARG, "%s: null pointer", who);
    const uint64_t outs_off = (uint64_t(table_bytes) + 255) / 256 * 256;
    const uint64_t need = outs_off + 8 * uint64_t(n_outs);
    if (table_bytes > ST_NOALLOC_SCRATCH_BYTES || need > ST_NOALLOC_SCRATCH_BYTES)
        return st_fail(ST_E_ARG, "%s: a %zu-byte work table and %zu output pointers need %llu bytes of scratch, at most %u",
                       who, table_bytes, n_outs, (unsigned long long)need, unsigned(ST_NOALLOC_SCRATCH_BYTES));
    if (table_bytes < sizeof(st_table_header)) return st_fail(ST_E_ARG, "%s: %zu-byte work table has no header", who, table_bytes);
    st_table_header h;
    memcpy(&h, table_host, sizeof h);
    const uint64_t groups = (uint64_t(n) + ST_UNITS_PER_GROUP - 1) / ST_UNITS_PER_GROUP;
    if (h.magic != ST_TABLE_MAGIC || h.bytes != table_bytes || h.map_offset != sizeof(st_table_header) ||
        h.desc_offset != stk::table_desc_offset(groups) || h.desc_offset + 64 * uint64_t(h.n_desc) > table_bytes)
        return st_fail(ST_E_ARG, "%s: not a work table of %zu bytes and %zu units", who, table_bytes, n);
    if (h.units != n) return st_fail(ST_E_ARG, "%s: the table holds %llu work units, n is %zu", who, (unsigned long long)h.units, n);
    if (h.out_dtype != out_dtype)
        return st_fail(ST_E_ARG, "%s: the table was planned for output type %u, the launch asks for %u", who, h.out_dtype, out_dtype);
    const uint8_t* descs = static_cast<const uint8_t*>(table_host) + h.desc_offset;
    for (uint32_t d = 0; d < h.n_desc; ++d) {
        uint32_t out;
        memcpy(&out, descs + 64 * size_t(d) + offsetof(st_desc, out), sizeof out);
        if (out >= n_outs) return st_fail(ST_E_ARG, "%s: descriptor %u writes output %u of %zu", who, d, out, n_outs);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = -1;
    if (hipStreamGetDevice(s, &dev) != hipSuccess) return st_fail(ST_E_HIP, "%s: hipStreamGetDevice failed", who);
    uint8_t* ptr = nullptr;
    st_status r = scratch_address(dev, &ptr);
    if (r != ST_OK) return r;
    // Every byte the kernel reads is written by these two copies; nothing needs clearing.
    if (hipMemcpyAsync(ptr, table_host, table_bytes, hipMemcpyHostToDevice, s) != hipSuccess ||
        (n_outs && hipMemcpyAsync(ptr + outs_off, outs_host, 8 * n_outs, hipMemcpyHostToDevice, s) != hipSuccess))
        return st_fail(ST_E_HIP, "%s: copy into the scratch array failed", who);
    if (h.flags & ST_TABLE_STREAM_STORES) flags |= ST_MAT_STREAM_STORES;  // the header's store policy
    return st_materialize_as(blob, ptr, n, reinterpret_cast<void* const*>(ptr + outs_off), out_dtype, flags, stream);
}

extern "C" st_status st_materialize(const void* blob, const void* descs, size_t n, void* const* outs, void* stream) {
    return st_materialize_as(blob, descs, n, outs, ST_OUT_BF16, 0, stream);
}

extern "C" st_status st_materialize_slices(const void* blob, const void* descs, size_t n, void* const* outs,
                                           void* stream) {
    return st_materialize_as(blob, descs, n, outs, ST_OUT_BF16, ST_MAT_SLICES, stream);
}
