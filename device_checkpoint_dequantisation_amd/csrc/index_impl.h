// Host-side internals of the safetensors index, shared by the header index (index.cpp), the
// streaming planner (stream_plan.cpp) and the staging code (stage.cpp).
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

#include "st_internal.h"

namespace sti {

struct Tensor {
    std::string name;
    int dtype;
    std::vector<int64_t> shape;
    uint64_t begin, end;
    uint64_t numel;
};

struct Output {
    uint32_t tensor;
    int64_t scale = -1, scale2 = -1;
    st_kind kind;
    std::vector<int64_t> shape;
    uint64_t numel;
};

// Work table for outputs sel[0..k): header, the map from each group of ST_UNITS_PER_GROUP units to
// the descriptor holding its first unit, and the descriptors (descriptor j writes outs[j]).
// at[t], if given, is the device-blob offset of tensor t's bytes (default: its data-section
// offset).  Throws std::length_error at 2^32 or more work units, std::bad_alloc when out of memory.
std::vector<unsigned char> build_table(const st_index& ix, const uint32_t* sel, size_t k, uint64_t* units_out,
                                       const uint64_t* at = nullptr);

// Clears this thread's st_last_error() message.
void clear_error();

}  // namespace sti

// True if `plan` was built from `idx` (st_stream_plan_build).
bool st_stream_plan_of(const st_stream_plan* plan, const st_index* idx);

struct st_index {
    uint64_t header_len = 0;   // N
    uint64_t data_size = 0;
    std::string metadata_json = "{}";
    std::vector<sti::Tensor> tensors;
    std::unordered_map<std::string, uint32_t> by_name;
    std::vector<sti::Output> outputs;
    std::vector<uint64_t> out_offset;  // arena offsets
    uint64_t arena_bytes = 0;
    std::vector<unsigned char> table;  // header, group map, descriptors
    uint64_t total_units = 0;
    uint32_t unit_log2_scale = 0;
    uint32_t out_dtype = ST_OUT_BF16;  // st_out_dtype of every output
};

namespace sti {
// Bytes per output element.
inline uint64_t out_bytes(const st_index& ix) { return ix.out_dtype == ST_OUT_F32 ? 4 : 2; }
}  // namespace sti
