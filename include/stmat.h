/*
 * stmat — materialise safetensors checkpoint weights as bf16 on an MI355X (gfx950).
 *
 * C ABI of libstmat.so.  Plain pointers and sizes only; no C++ or framework types cross it.
 * Streams and events are HIP handles (hipStream_t / hipEvent_t) passed as void*.
 *
 * The operation.  The pages ("Disk tier safetensors streaming design audit", sections
 * "FastSageTensors capability audit" and "Strategy summary") describe a metadata-only index
 * of a safetensors file (per tensor: dtype, shape, data_offsets; no tensor bytes read) and range
 * reads of tensor bytes into pinned host memory followed by a copy to the GPU.  The serving
 * document ("Resident Modal LLM Architecture", section "Current Backend Boundary") names the
 * quantised checkpoint families whose weights must be turned into compute-dtype tensors: Qwen
 * block-FP8 and NVIDIA ModelOpt NVFP4; the design audit ("Mandatory research audit") names
 * ComfyUI's scaled-FP8 checkpoints.  This library implements that path:
 *
 *   st_index_build / st_index_open   header bytes -> index (host, metadata only)
 *   st_stage_file                    file byte ranges -> pinned ring -> device blob (side stream)
 *   st_stream_plan_build/st_stream_file  staging steps, each decoded as soon as its bytes land
 *   st_materialize                   device blob + work table -> bf16 outputs (one launch)
 *
 * Output element values (bit-exact definition; rounding is IEEE binary32 round-to-nearest-even
 * for every multiply, then round-to-nearest-even to bfloat16; any NaN result is 0x7FC0;
 * no subnormal flushing):
 *   PASS_BF16     bf16 input bits copied unchanged
 *   CAST_F16      bf16(float(h))
 *   CAST_F32      bf16(x)
 *   FP8_TENSOR    bf16(e4m3(w) * s)                 X.weight F8_E4M3 + X.scale_weight F32 []
 *   FP8_BLOCK128  bf16(e4m3(w[i,j]) * S[i/128,j/128]) X.weight F8_E4M3 [M,N] +
 *                                                  X.weight_scale_inv F32 [ceil(M/128),ceil(N/128)]
 *   NVFP4         bf16((e2m1(q[i,j]) * e4m3(bs[i,j/16])) * g)
 *                 X.weight U8 [M,K/2] (element 2k in the low nibble of byte k) or F4 [M,K] +
 *                 X.weight_scale F8_E4M3 [M,K/16] + X.weight_scale_2 F32 []
 *   MXFP8         bf16(e4m3(w[i,j]) * e8m0(s[i,j/32]))  X.weight F8_E4M3 [M,K] +
 *                                                  X.weight_scale F8_E8M0 [M,K/32]
 *   MXFP4         bf16(e2m1(q[i,j]) * e8m0(s[i,j/32]))  X.weight U8 [M,K/2] or F4 [M,K] +
 *                                                  X.weight_scale F8_E8M0 [M,K/32]
 * e4m3 is OCP E4M3 "fn" (bias 7, no infinities, NaN at S.1111.111); e2m1 is OCP-MX E2M1; e8m0 is
 * the OCP Microscaling scale 2^(e-127), NaN at 0xFF (the formats of the OCP Microscaling
 * specification: 32 consecutive elements of a row share a scale; K must be a multiple of 32).
 *
 * Errors.  Every call returns ST_OK (0) or a negative st_status; nothing throws across the ABI.
 * st_last_error() then names the tensor, the field and the measured values.
 */
#ifndef STMAT_H
#define STMAT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum st_status {
    ST_OK = 0,
    ST_E_ARG = -1,      /* null pointer, size too small, bad option */
    ST_E_IO = -2,       /* open/read/stat failed, file shorter than the header says */
    ST_E_HEADER = -3,   /* header length field: too short, over the cap, past end of file, not UTF-8 */
    ST_E_JSON = -4,     /* header is not a JSON object, duplicate key, bad string */
    ST_E_DTYPE = -5,    /* unknown dtype, or a dtype that cannot be materialised */
    ST_E_SHAPE = -6,    /* bad shape, span != numel * itemsize, rank, NVFP4 K % 16, size limits */
    ST_E_OFFSETS = -7,  /* offsets overlap, leave a gap, or do not end at the end of the file */
    ST_E_SCALE = -8,    /* missing, orphaned, ambiguous or mis-shaped scale tensor */
    ST_E_NOMEM = -9,    /* host allocation failed */
    ST_E_HIP = -10      /* a HIP runtime call failed (launch, copy, event) */
} st_status;

/* safetensors dtype strings, in this order: BOOL U8 I8 F8_E4M3 F8_E5M2 F8_E8M0 I16 U16 F16
 * BF16 I32 U32 F32 I64 U64 F64 F4 F6_E2M3 F6_E3M2 */
typedef enum st_dtype {
    ST_DT_BOOL = 0, ST_DT_U8, ST_DT_I8, ST_DT_F8_E4M3, ST_DT_F8_E5M2, ST_DT_F8_E8M0,
    ST_DT_I16, ST_DT_U16, ST_DT_F16, ST_DT_BF16, ST_DT_I32, ST_DT_U32, ST_DT_F32,
    ST_DT_I64, ST_DT_U64, ST_DT_F64, ST_DT_F4, ST_DT_F6_E2M3, ST_DT_F6_E3M2
} st_dtype;

typedef enum st_kind {
    ST_KIND_PASS_BF16 = 0, ST_KIND_CAST_F16 = 1, ST_KIND_CAST_F32 = 2,
    ST_KIND_FP8_TENSOR = 3, ST_KIND_FP8_BLOCK128 = 4, ST_KIND_NVFP4 = 5,
    ST_KIND_MXFP8 = 6, ST_KIND_MXFP4 = 7
} st_kind;

/* Output element type, chosen per index (st_plan_opts.flags).  Every output element is the fp32
 * result of its definition rounded to nearest-even in this type (fp32: the result itself); any NaN
 * becomes the type's canonical quiet NaN (bf16 0x7FC0, fp16 0x7E00, fp32 0x7FC00000); no
 * subnormal flushing.  A bf16 source copied to a bf16 output keeps its bits. */
typedef enum st_out_dtype { ST_OUT_BF16 = 0, ST_OUT_F16 = 1, ST_OUT_F32 = 2 } st_out_dtype;

#define ST_MAX_NDIM 8
#define ST_HEADER_CAP 100000000ull   /* largest accepted JSON header, bytes */
#define ST_BLOB_ALIGN 256            /* required alignment of the device blob */
#define ST_OUT_ALIGN 16              /* required alignment of every output pointer */

/* One header entry (a tensor as stored).  begin/end are relative to the data section. */
typedef struct st_tensor_meta {
    const char* name;        /* NUL-terminated UTF-8, valid for the index's lifetime */
    int32_t dtype;           /* st_dtype */
    int32_t ndim;
    int64_t shape[ST_MAX_NDIM];
    uint64_t begin, end;
} st_tensor_meta;

/* One bf16 output (a weight after scale pairing), in output order. */
typedef struct st_output_info {
    const char* name;        /* the weight tensor's name */
    int32_t kind;            /* st_kind */
    int32_t ndim;
    int64_t shape[ST_MAX_NDIM];  /* logical bf16 shape (NVFP4: [M, K]) */
    uint64_t numel;
    int64_t tensor;          /* header-entry index of the weight */
    int64_t scale;           /* header-entry index of its scale tensor, or -1 */
    int64_t scale2;          /* header-entry index of the NVFP4 global scale, or -1 */
} st_output_info;

/* The device work table, built on the host by the library and uploaded by the caller as one
 * block of device memory (64-byte aligned):
 *
 *   st_table_header                      64 bytes
 *   uint32_t map[groups]                 at offset 64: for every group of 4 consecutive work units
 *                                        (groups = ceil(units / 4)), the descriptor that holds the
 *                                        group's first unit; padded to a multiple of 64 bytes
 *   st_desc[n_desc]                      one 64-byte descriptor per output, at desc_offset =
 *                                        64 + round_up(4 * groups, 64)
 *
 * A work unit is 2^unit_shift consecutive output elements of one output; an output of numel
 * elements has ceil(numel / 2^unit_shift) units, numbered in output order from unit_begin.
 * The kernel runs one 64-lane wavefront per unit and one 4-wave workgroup per map entry.
 * Offsets in descriptors are bytes from the start of the blob (= the file's data section). */
#define ST_TABLE_MAGIC 0x334D5453u   /* "STM3" */
#define ST_UNITS_PER_GROUP 4

typedef struct st_table_header {
    uint32_t magic;          /* ST_TABLE_MAGIC */
    uint32_t n_desc;         /* descriptors */
    uint64_t units;          /* work units (below 2^32) */
    uint64_t desc_offset;    /* bytes from the table start to st_desc[0] */
    uint64_t map_offset;     /* bytes from the table start to map[0] (always 64) */
    uint64_t bytes;          /* size of the whole table */
    uint32_t out_dtype;      /* st_out_dtype the outputs were planned for */
    uint32_t flags;          /* ST_TABLE_STREAM_STORES, or 0 */
    uint64_t reserved[2];
} st_table_header;           /* 64 bytes */
/* st_table_header.flags: the table's outputs are larger than the GPU's last-level (Infinity) cache
 * (256 MiB on MI355X), so they are better written with non-temporal stores than kept there: a
 * caller that holds the table passes ST_MAT_STREAM_STORES to st_materialize_as when it is set
 * (st_stream_file and st_materialize_noalloc read it themselves).  Set by the planner. */
#define ST_TABLE_STREAM_STORES 1u

typedef struct st_desc {
    uint64_t src;            /* weight bytes */
    uint64_t scale;          /* FP8_TENSOR fp32 scale / FP8_BLOCK128 fp32 grid / NVFP4 e4m3 block scales */
    uint64_t scale2;         /* NVFP4 fp32 global scale */
    uint32_t pitch;          /* column slice: source elements from one output row to the next
                                (the full row length); 0 = the output's source is contiguous */
    uint32_t flags;          /* ST_DESC_EXACT: every element takes the exact per-element path */
    uint32_t unit_begin;     /* this output's first work unit in the table */
    uint32_t unit_end;       /* one past its last work unit */
    uint32_t tail;           /* elements in its last unit (1 .. 2^unit_shift) */
    uint32_t out;            /* index into the outs[] pointer array */
    uint32_t cols;           /* FP8_BLOCK128: N, NVFP4: K, a column slice: its width; otherwise 0 */
    uint32_t grid_cols;      /* FP8_BLOCK128: ceil(N / 128) of the whole tensor */
    uint32_t div_magic;      /* FP8_BLOCK128 or a column slice: multiplier of the exact division
                                by cols */
    uint32_t meta;           /* st_kind | unit_shift << 8 | div_shift << 16 (a unit is
                                2^unit_shift elements; div_shift goes with div_magic) */
} st_desc;                   /* 64 bytes */
#define ST_DESC_EXACT 1u     /* st_desc.flags */
/* st_desc.flags: a split descriptor decodes every column shard of some rows of one output at once:
 * the source rows are read whole (pitch = their length C), cut into 2^grid_cols shards of cols
 * elements each, and shard s is written to outs[out + s] as a [rows, cols] row-major array.  Planned
 * by st_index_table_slices for a request that lists all column shards of an NVFP4 or MXFP4 weight
 * in column order; other kinds take the per-element path for it. */
#define ST_DESC_SPLIT 2u

/* Planning options; pass NULL for the defaults. */
typedef struct st_plan_opts {
    uint32_t unit_log2_scale;  /* work unit = (kind's default unit) << this; 0..6, default 0 */
    uint32_t flags;            /* bits 0-1: st_out_dtype of every output (default ST_OUT_BF16);
                                  the other bits must be 0 */
} st_plan_opts;

typedef struct st_index st_index;   /* opaque, host memory, owned by the library */

/* Human-readable description of the last error on the calling thread ("" if none).  Valid
 * until the next stmat call on the same thread.  Messages name the tensor, the field and the
 * measured values: the pages' loader fails with the measured free and total memory rather than
 * attempting an unsafe load ("Resident Modal LLM Architecture", "Residency And Memory") and stops
 * with a hard error that says what to change when a requested read path is unavailable ("Disk
 * tier safetensors streaming design audit", "Strategy summary / Range reads and tiering"). */
const char* st_last_error(void);

/* From the first 8 bytes of a file, the number of bytes the header occupies (8 + N).
 * Fails with ST_E_HEADER if N exceeds ST_HEADER_CAP.  The header alone carries every tensor's
 * dtype, shape and data offsets ("Disk tier safetensors streaming design audit", "FastSageTensors
 * capability audit": header parsing and metadata); this is how much of the file to read for it. */
st_status st_header_size(const void* first8, uint64_t* header_bytes);

/* Build the metadata-only index from the first header_len bytes of a safetensors file of
 * file_size bytes (header_len >= 8 + N; extra bytes are ignored).  Parses and validates the
 * header, checks that the data_offsets tile the data section exactly, pairs quantised weights
 * with their scales, and plans the device descriptor table.  No tensor byte is read.
 * Fails (and sets *out = NULL) on any malformed header; see st_status.
 * Source: the SafeTensorIndex / TensorMeta of "Disk tier safetensors streaming design audit",
 * "Strategy summary / Streaming safetensors mapping" (metadata-only parsing, no full dict
 * materialisation); the scale pairing covers the checkpoint families of "Resident Modal LLM
 * Architecture", "Current Backend Boundary" (Qwen block-FP8, ModelOpt NVFP4) and the scaled-FP8
 * conversion of the design audit's "Mandatory research audit". */
st_status st_index_build(const void* header_bytes, uint64_t header_len, uint64_t file_size,
                         const st_plan_opts* opts, st_index** out);

/* st_index_build on the header of the file at `path` (reads only 8 + N bytes).  ST_E_IO if the
 * file cannot be opened or read.  Source: as st_index_build (metadata read without loading a
 * tensor). */
st_status st_index_open(const char* path, const st_plan_opts* opts, st_index** out);

/* Frees an index and everything it owns (names, tables); NULL is a no-op. */
void st_index_free(st_index* idx);

/* The byte ranges a load reads: only the data section, never the header twice ("Disk tier
 * safetensors streaming design audit", "Strategy summary / Range reads and tiering": read only
 * the tensor range).  Both return 0 for a NULL index. */
uint64_t st_index_data_offset(const st_index* idx);   /* 8 + N: file offset of the data section */
uint64_t st_index_data_size(const st_index* idx);     /* bytes of the data section */
/* Bytes to allocate for the device blob: data size plus 64, rounded up to a multiple of 256.
 * The kernel reads whole aligned words, which may reach a few bytes past the data, so the
 * padding must be present. */
uint64_t st_index_blob_bytes(const st_index* idx);
/* Header entries, read from the metadata alone: per tensor its name, dtype, shape and data
 * offsets ("Disk tier safetensors streaming design audit", "FastSageTensors capability audit":
 * a per-tensor frame of dtype, shape and data_offsets with no tensor allocated; "Strategy
 * summary / Streaming safetensors mapping": metadata-only keys).  st_index_tensor fails with
 * ST_E_ARG for a NULL pointer or i >= st_index_count. */
size_t st_index_count(const st_index* idx);           /* header entries (tensors) */
st_status st_index_tensor(const st_index* idx, size_t i, st_tensor_meta* out);
/* Index of the header entry called `name`, or -1. */
int64_t st_index_find(const st_index* idx, const char* name);
/* The header's __metadata__ as a JSON object text ("{}" if absent); valid for the index's lifetime.
 * The design audit asks for metadata returned without loading tensors ("Disk tier safetensors
 * streaming design audit", "Pipeline refactors"). */
const char* st_index_metadata_json(const st_index* idx);

/* The outputs: every weight after scale pairing, with its kind (bf16 copy, fp16/fp32 cast,
 * scaled FP8, block FP8, NVFP4, MXFP8, MXFP4) and logical shape, in output order.  The quantised
 * kinds are the checkpoint families of "Resident Modal LLM Architecture", "Current Backend
 * Boundary" and of the design audit's "Mandatory research audit".  st_index_output fails with
 * ST_E_ARG for a NULL pointer or k >= st_index_num_outputs. */
size_t st_index_num_outputs(const st_index* idx);
st_status st_index_output(const st_index* idx, size_t k, st_output_info* out);
/* The output element type the index plans for (st_plan_opts.flags). */
uint32_t st_index_out_dtype(const st_index* idx);
/* Byte offset of output k inside one output arena in which every output starts on a
 * 256-byte boundary, and the arena's total size (2 or 4 bytes per element).  The arena is
 * framework-allocated memory that the outputs view ("Disk tier safetensors streaming design
 * audit", "FastSageTensors capability audit": torch interop allocates tensor memory and wraps raw
 * pointers as tensors).  0 for a NULL index or k out of range. */
uint64_t st_index_output_offset(const st_index* idx, size_t k);
uint64_t st_index_output_arena_bytes(const st_index* idx);
/* Bytes read + bytes written by materialising every output (the data section plus 2 or 4
 * bytes per output element): the byte count a throughput figure for the decode divides.  The
 * pages publish no such figure; this is the algorithmic traffic, not a counter reading. */
uint64_t st_index_traffic_bytes(const st_index* idx);
/* Device memory the whole load needs: blob + work table + pointer array + arena.
 * Compare with the free device memory before allocating; the requirement is arithmetic.  The
 * pages' loader checks the free memory before a load and fails with the measured free and total
 * figures ("Resident Modal LLM Architecture", "Residency And Memory"), and decides admission by
 * arithmetic it owns ("VRAM co-management across processes", "The WDDM position", current
 * position).  0 for a NULL index. */
uint64_t st_index_device_bytes(const st_index* idx);

/* The work table for every output (descriptor k writes outs[k]), host memory owned by the
 * index.  *bytes = table size, *units = work units (the `n` st_materialize takes); either
 * pointer may be NULL.  NULL for a NULL index.  Source: the descriptor table the metadata-only
 * index hands to the device ("Disk tier safetensors streaming design audit", "Strategy summary /
 * Streaming safetensors mapping"). */
const void* st_index_table(const st_index* idx, size_t* bytes, uint64_t* units);
/* The same table as st_index_table, in the argument order (index, n, bytes): *n receives the
 * table's work-unit count, the `n` that st_materialize takes (the launch is one wavefront per
 * unit, so a unit count, not a descriptor count, sizes it); *bytes the table size.  Either
 * pointer may be NULL; NULL for a NULL index. */
const void* st_index_descs(const st_index* idx, size_t* n, size_t* bytes);

/* A self-contained work table for a subset of outputs: sel[0..k) are output indices (any
 * order; repeats allowed); descriptor j writes outs[j], so outs[j] must point to output sel[j].
 * With dst == NULL only *bytes and *units are set (a size query); otherwise dst_bytes must be
 * at least that size.  ST_E_ARG for an index out of range or dst too small.  Used for on-demand
 * loads of single tensors ("Disk tier safetensors streaming design audit", "Strategy summary /
 * Streaming safetensors mapping": loading tensors on demand; "Tests and docs": single-tensor
 * loading). */
st_status st_index_table_subset(const st_index* idx, const uint32_t* sel, size_t k, void* dst,
                                size_t dst_bytes, size_t* bytes, uint64_t* units);

/* ---- Sliced materialisation (tensor-parallel shards) ---------------------------------------------
 * A slice is a block of rows and columns of one output, seen as a matrix: an output of shape
 * [d0, d1, ...] is [d0, d1 * d2 * ...] (a 1-d output [n] is [n, 1], a scalar [1, 1]).  Slice j
 * materialises rows [row_begin, row_end) and columns [col_begin, col_end) as one contiguous
 * row-major bf16 array of (row_end - row_begin) * (col_end - col_begin) elements, written to
 * outs[j]; its values are exactly the corresponding elements of the whole output.  Row slices keep
 * the source contiguous; column slices read every source row at a pitch (the pages name tensor
 * slicing among the metadata an index must carry: "FastSageTensors capability audit").
 * Cuts respect the scale blocks: FP8_BLOCK128 row_begin and col_begin are multiples of 128; NVFP4
 * col_begin and the slice width are multiples of 16.  A column slice needs fewer than 2^32 output
 * elements and a row length below 2^32.  Column slices whose chunks would cross rows or lose a
 * common alignment take the exact per-element path (correct, slower). */
typedef struct {
    uint32_t output;         /* output index */
    uint32_t reserved;       /* 0 */
    int64_t row_begin, row_end;   /* row_end < 0: to the last row */
    int64_t col_begin, col_end;   /* col_end < 0: to the last column */
} st_slice;

/* Work table for slices[0..k) over the data-section blob; slice j is written to outs[j].  Same
 * size-query convention as st_index_table_subset.  ST_E_ARG for an out-of-range output or
 * bounds, ST_E_SHAPE for a cut that splits a scale block or a column slice too large.
 * Planning: consecutive slices that are every column shard of the same rows of one NVFP4 or MXFP4
 * output (2, 4, ... 64 shards of equal width, in column order, each below 2^32 bytes) become one
 * ST_DESC_SPLIT descriptor that reads those rows whole; other column slices of
 * packed-fp4 outputs that share rows are interleaved in bands of work units so that they read the
 * rows' shared cache lines together; every other slice keeps its own descriptor in request order,
 * except that when the descriptors' bytes fall unevenly on the GPU's eight XCDs (each takes one
 * contiguous eighth of the work units), slices of 16,384 units or more are cut into eight pieces,
 * one per eighth. */
st_status st_index_table_slices(const st_index* idx, const st_slice* slices, size_t k, void* dst,
                                size_t dst_bytes, size_t* bytes, uint64_t* units);
/* Elements of slice `s` once its bounds are resolved (rows * cols), or ST_E_ARG.  Source: as the
 * slices above (slicing metadata). */
st_status st_index_slice_numel(const st_index* idx, const st_slice* s, uint64_t* rows, uint64_t* cols);

/* Stage the data section of the file at `path` into `blob_dev` (device memory of at least
 * st_index_blob_bytes bytes, ST_BLOB_ALIGN-aligned).  Reads the file in chunks into the
 * caller's pinned host buffer `pinned` (pinned_bytes >= 2 MiB; it is split into a ring of
 * chunks) and copies each chunk with hipMemcpyAsync on `side_stream`; records `done_event`
 * (may be NULL) on that stream after the last copy.  Returns once every read is done and every
 * copy is enqueued; the pinned buffer must stay allocated until done_event completes.
 * A later st_stage_file or st_stream_file call given the same pinned buffer first waits (on the
 * host) for this call's copies out of it, so a caller may reuse the buffer at once.
 * If `seconds_read` is not NULL it receives
 * the wall time spent in file reads (for a file -> pinned rate).
 * Errors: ST_E_ARG (null pointers, pinned buffer too small, misaligned blob), ST_E_IO (open, size
 * or read failure), ST_E_HIP (a copy or event).
 * Source: "Disk tier safetensors streaming design audit", "Strategy summary / Range reads and
 * tiering" (Disk->RAM->GPU: read the range into pinned CPU memory, copy it to the GPU). */
st_status st_stage_file(const char* path, const st_index* idx, void* blob_dev, void* pinned,
                        size_t pinned_bytes, void* side_stream, void* done_event,
                        double* seconds_read);

/* ---- Streaming plans: range reads, copies and decoding in flight together ----------------------
 * The pages' disk tier reads only the byte ranges a load needs into pinned host memory, copies
 * them to the GPU and then releases the host buffer; a state dict loads tensors on demand and a RAM
 * tier keeps recently read weights ("Disk tier safetensors streaming design audit", "Strategy
 * summary / Range reads and tiering", "Disk tier integration").  A stream plan covers every output
 * of a checkpoint (st_stream_plan_build) or a chosen set (st_stream_plan_select).  It reads the
 * outputs' weight and scale tensors, as runs of file-adjacent tensors, and cuts them into
 * staging steps of at most chunk_bytes.  Bytes are staged in file order, except that a scale
 * tensor lying more than one chunk past the end of its weight is staged first (checkpoints that
 * keep all scales at the end).  Each step carries a work table for the outputs whose inputs have
 * all been copied once the step's copies are done.  The device blob is either laid out like the
 * data section (st_index_blob_bytes) or, with ST_PLAN_PACK, compact: only the plan's runs, each
 * starting on a 256-byte boundary plus its data-section offset mod 256 (so the kernel sees the
 * same alignment).  st_stream_file reads, copies and decodes step by step, so decoding overlaps
 * the reads and copies of later steps; st_read_plan reads a plan's bytes into host memory. */

typedef struct st_stream_plan st_stream_plan;  /* opaque, host memory, library-owned */

typedef struct {
    uint64_t begin, end;    /* bytes [begin, end) of the data section */
    uint64_t dst;           /* byte offset in the plan's device blob where they go */
    uint32_t step;          /* the staging step that copies them */
    uint32_t reserved;
} st_stream_range;

#define ST_PLAN_PACK 1u     /* st_stream_plan_select: compact blob of only the selected inputs */

typedef struct {
    uint64_t bytes;         /* bytes this step copies */
    uint32_t first_range;   /* its ranges: st_stream_plan_ranges()[first_range .. + n_ranges) */
    uint32_t n_ranges;
    uint32_t first_out;     /* outputs it completes: st_stream_plan_order()[first_out .. + n_out) */
    uint32_t n_out;
    uint64_t table_offset;  /* byte offset of its work table in st_stream_plan_tables (64-B aligned) */
    uint64_t units;         /* that table's work-unit count; 0 = nothing to decode */
} st_stream_step;

/* Plan the streaming load of every output of `idx` in steps of at most chunk_bytes (>= 64 KiB).
 * Every byte of the data section belongs to exactly one range; every output to exactly one step;
 * the blob is laid out like the data section.  ST_E_ARG for a NULL index or a chunk too small.
 * Source: the range reads and tiering cited above this group. */
st_status st_stream_plan_build(const st_index* idx, uint64_t chunk_bytes, st_stream_plan** out);
/* Plan the load of outputs sel[0..k) (distinct indices) only: the ranges cover their weight and
 * scale tensors (plus gaps of at most 4 KiB between file-adjacent ones).  flags: 0 or
 * ST_PLAN_PACK.  Output order within a step follows sel. */
st_status st_stream_plan_select(const st_index* idx, const uint32_t* sel, size_t k, uint64_t chunk_bytes,
                                uint32_t flags, st_stream_plan** out);
/* Accessors of a plan (the plan owns what they return; 0 / NULL for a NULL plan).  Source: the
 * range reads and tiering cited above this group. */
void      st_stream_plan_free(st_stream_plan* plan);
uint64_t  st_stream_plan_chunk_bytes(const st_stream_plan* plan);
/* Bytes of the device blob the plan's tables address (ST_BLOB_ALIGN-aligned allocation). */
uint64_t  st_stream_plan_blob_bytes(const st_stream_plan* plan);
size_t    st_stream_plan_num_steps(const st_stream_plan* plan);
st_status st_stream_plan_step(const st_stream_plan* plan, size_t s, st_stream_step* out);
/* All ranges, step-major; valid for the plan's lifetime. */
const st_stream_range* st_stream_plan_ranges(const st_stream_plan* plan, size_t* n);
/* Output indices in plan order (step-major); entry j of the `outs_dev` array passed to
 * st_stream_file must point to output order[j]. */
const uint32_t* st_stream_plan_order(const st_stream_plan* plan, size_t* n);
/* Every step's work table, concatenated (host memory; upload once to a 64-byte aligned device
 * buffer for st_stream_file). */
const void* st_stream_plan_tables(const st_stream_plan* plan, size_t* bytes);

typedef struct {
    double seconds_read;    /* wall time in file reads */
    double seconds_wait;    /* wall time waiting for a ring slot's previous copy */
    uint64_t bytes_read;
    uint32_t steps;         /* steps staged */
    uint32_t launches;      /* st_materialize launches enqueued */
    double seconds_first_launch;  /* wall time from the call's start until the first decode was
                                     enqueued (its step's bytes read and their copy queued); -1 if
                                     there was none */
} st_stream_stats;

/* Stream the file at `path` through `plan`: for each step, read its ranges into a slot of the
 * pinned ring (pinned_bytes >= 4 * chunk_bytes; four slots), copy each to blob_dev + dst with
 * hipMemcpyAsync on `side_stream`, make `compute_stream` wait for those copies and enqueue
 * st_materialize over the step's table on `compute_stream`.  A later call given the same pinned
 * buffer first waits (on the host) for this call's copies out of it.
 *   blob_dev    st_stream_plan_blob_bytes bytes, ST_BLOB_ALIGN-aligned
 *   tables_dev  device copy of st_stream_plan_tables, 64-byte aligned
 *   outs_dev    device array of output pointers in plan order (see st_stream_plan_order)
 *   done_event  (may be NULL) recorded on compute_stream after the last launch: once it has
 *               completed, every output is decoded and the pinned buffer is free.
 * Returns once every read is done and every copy and launch is enqueued.  The library allocates no
 * device memory and synchronises no stream (it waits on its own ring events before reusing a
 * slot).  Errors: ST_E_ARG (null pointers, pinned buffer too small, plan of another index,
 * misaligned buffers), ST_E_IO (open, size or read failure), ST_E_HIP (a copy, event or launch);
 * after an error the side stream has been synchronised so the ring is no longer read. */
st_status st_stream_file(const char* path, const st_index* idx, const st_stream_plan* plan, void* blob_dev,
                         const void* tables_dev, void* const* outs_dev, void* pinned, size_t pinned_bytes,
                         void* side_stream, void* compute_stream, void* done_event, st_stream_stats* stats);

/* Read every range of `plan` from the file at `path` into host memory: range r lands at
 * host_blob + dst.  host_bytes must be at least st_stream_plan_blob_bytes(plan); bytes no range
 * covers are left as they are.  Uploading host_blob (one copy) and launching the plan's tables
 * then decodes the plan's outputs without touching the file again (a RAM tier: "Disk tier
 * safetensors streaming design audit", "Disk tier integration", an LRU of RAM-resident weights
 * with a byte limit).  Synchronous; no GPU calls.  If `seconds_read` is not NULL it receives the
 * wall time of the reads.  Errors: ST_E_ARG (null pointers, buffer too small, plan of another
 * index), ST_E_IO (open, size or read failure). */
st_status st_read_plan(const char* path, const st_index* idx, const st_stream_plan* plan, void* host_blob,
                       size_t host_bytes, double* seconds_read);
/* st_read_plan for n plans of the same index at once (one pool of reader threads): plan j's
 * ranges land in host_blobs[j], which holds host_bytes[j] bytes. */
st_status st_read_plans(const char* path, const st_index* idx, const st_stream_plan* const* plans,
                        void* const* host_blobs, const size_t* host_bytes, size_t n, double* seconds_read);

/* Enqueue the grouped materialise kernel on `stream` (hipStream_t; NULL = default stream).
 * It turns the staged bytes of every descriptor into compute-dtype tensors: the checkpoint
 * families of "Resident Modal LLM Architecture", "Current Backend Boundary" (Qwen block-FP8,
 * ModelOpt NVFP4) and the scaled-FP8 checkpoints of the design audit's "Mandatory research
 * audit", each element as defined at the top of this header.
 *   blob   device copy of the data section (st_index_blob_bytes bytes, ST_BLOB_ALIGN-aligned)
 *   descs  device copy of a work table (st_index_table / st_index_table_subset), 64-byte aligned
 *   n      the table's work-unit count (returned with the table); the launch is one 64-lane
 *          wavefront per unit, so n decides the grid.  A value that disagrees with the table's
 *          header makes every wavefront return without writing.
 *   outs   device array of bf16 output pointers, each ST_OUT_ALIGN-aligned and large enough
 *          for its output's numel elements; descriptor d writes outs[desc[d].out]
 * One launch covers every descriptor.  Only enqueues: it never allocates, copies or
 * synchronises; kernel faults surface at the caller's next synchronisation.  Returns ST_E_ARG
 * for null pointers or misaligned blob/table (n > 0) and ST_E_HIP if the launch fails.
 * n == 0 is a no-op. */
st_status st_materialize(const void* blob, const void* descs, size_t n, void* const* outs,
                         void* stream);

/* st_materialize for tables that hold column slices (st_index_table_slices): the same arguments
 * and results, with column slices on the strided fast path.  st_materialize decodes such tables
 * correctly too, one element at a time; this entry point is a separate kernel so that the
 * whole-output kernel carries no strided code. */
st_status st_materialize_slices(const void* blob, const void* descs, size_t n, void* const* outs,
                                void* stream);

#define ST_MAT_SLICES 1u     /* st_materialize_as: the instance with the strided column-slice path */
/* st_materialize_as: stream the outputs past the caches (non-temporal, system-scope stores).  Pass
 * it when the table header carries ST_TABLE_STREAM_STORES (outputs larger than the last-level
 * cache): measured on MI355X, 2-4% on whole checkpoints and 7-11% on one rank's column shards; on
 * outputs that fit that cache, plain stores leave them there and measured faster. */
#define ST_MAT_STREAM_STORES 2u

/* The general entry point (source: as st_materialize): st_materialize for a table planned with
 * output type out_dtype
 * (st_out_dtype; outs then point to arrays of that type, aligned to it), flags 0 or a combination
 * of ST_MAT_SLICES and ST_MAT_STREAM_STORES.  One kernel instance per output type and flags: a
 * table planned for another type than
 * out_dtype makes every wavefront return without writing.  ST_E_ARG for an unknown type or
 * flag.  st_materialize = (ST_OUT_BF16, 0); st_materialize_slices = (ST_OUT_BF16, ST_MAT_SLICES). */
st_status st_materialize_as(const void* blob, const void* descs, size_t n, void* const* outs,
                            uint32_t out_dtype, uint32_t flags, void* stream);

/* ---- A launch that allocates nothing --------------------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  st_materialize_as takes its work table and output-pointer array
 * in device memory the caller allocated; this variant takes both in host memory and copies them
 * (hipMemcpyAsync on `stream`) into a device array the library owns, ST_NOALLOC_SCRATCH_BYTES per
 * GPU, held from the first call on a GPU until the process ends, then launches the same kernel on
 * it.  It calls no allocating routine.
 *   blob        the staged data section, as for st_materialize (device memory)
 *   table_host  a work table in host memory (st_index_table, st_index_descs, st_index_table_subset or
 *               st_index_table_slices), table_bytes long, n its work-unit count
 *   outs_host   host array of n_outs device output pointers (descriptor d writes outs_host[desc.out])
 *   out_dtype, flags  as st_materialize_as (ST_MAT_STREAM_STORES is added when the table header
 *               carries ST_TABLE_STREAM_STORES)
 * table_host and outs_host must stay valid and unchanged until `stream` has passed the launch (the
 * copies are asynchronous).  Limit: round_up(table_bytes, 256) + 8 * n_outs <= ST_NOALLOC_SCRATCH_BYTES
 * (the table takes 64 bytes per output plus 1 byte per work unit: about 32 G fp8 elements in one
 * call); larger loads split into subset tables.  Every call on one GPU shares that GPU's array:
 * calls on one stream are ordered, but calls that can overlap (other streams, other threads) race
 * and must be ordered by the caller.  The array keeps the last call's contents; nothing in it needs
 * clearing, since each call writes every byte its launch reads.
 * Errors: ST_E_ARG for null pointers, sizes past the limit, a table whose header disagrees with n,
 * table_bytes or out_dtype, or a descriptor naming an output pointer past n_outs (all checked on the
 * host before anything is enqueued); ST_E_HIP if the device lookup, a copy or the launch fails. */
#define ST_NOALLOC_SCRATCH_BYTES (32u << 20)
st_status st_materialize_noalloc(const void* blob, const void* table_host, size_t table_bytes, size_t n,
                                 void* const* outs_host, size_t n_outs, uint32_t out_dtype, uint32_t flags,
                                 void* stream);

#ifdef __cplusplus
}
#endif
#endif /* STMAT_H */
