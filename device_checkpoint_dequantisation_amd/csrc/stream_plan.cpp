// Streaming plan: staging steps over the data section and the outputs each step completes.
//
// The pages' disk tier reads only the byte ranges a load needs into pinned host memory, copies them
// to the GPU and releases the host buffer ("Disk tier safetensors streaming design audit",
// "Strategy summary / Range reads and tiering").  Here the data section is cut into staging steps
// of at most `chunk_bytes` each; an output is attached to the first step after which every byte of
// its weight and scale tensors is on the device, and each step carries a work table for just
// those outputs.  st_stream_file (stage.cpp) then reads, copies and decodes step by step, so the
// decoding of one step runs while later steps are read and copied.
//
// Order of the bytes.  In file order, except that a scale tensor lying more than one chunk past the
// end of its weight (a checkpoint that stores all scales at the end, say) is staged first, packed
// into the leading steps: otherwise none of those weights could be decoded before the file's end.
#include <algorithm>
#include <new>
#include <numeric>
#include <stdexcept>
#include <vector>

#include "index_impl.h"

struct st_stream_plan {
    const st_index* owner = nullptr;       // the index it was planned from
    uint64_t chunk_bytes = 0;
    std::vector<st_stream_range> ranges;   // step-major
    std::vector<st_stream_step> steps;
    std::vector<uint32_t> order;           // output indices, step-major
    std::vector<unsigned char> tables;     // every step's work table, each 64-byte aligned
};

namespace {

constexpr uint64_t kMinChunk = uint64_t(64) << 10;

// Appends the byte ranges [b, e) to the plan, opening a new step whenever the current one would
// exceed the chunk size.  `fill` is the byte count of the open step (-1: none open).
void add_bytes(st_stream_plan& p, uint64_t b, uint64_t e, int64_t& fill) {
    while (b < e) {
        if (fill < 0 || uint64_t(fill) == p.chunk_bytes) {
            st_stream_step s{};
            s.first_range = uint32_t(p.ranges.size());
            p.steps.push_back(s);
            fill = 0;
        }
        const uint64_t take = std::min<uint64_t>(e - b, p.chunk_bytes - uint64_t(fill));
        st_stream_step& s = p.steps.back();
        st_stream_range r{b, b + take, uint32_t(p.steps.size() - 1), 0};
        if (s.n_ranges && p.ranges.back().end == b) {
            p.ranges.back().end += take;  // contiguous with the step's previous range
        } else {
            p.ranges.push_back(r);
            ++s.n_ranges;
        }
        s.bytes += take;
        fill += int64_t(take);
        b += take;
    }
}

void build(const st_index& ix, st_stream_plan& p) {
    const size_t nt = ix.tensors.size(), no = ix.outputs.size();
    // scale tensors staged ahead of the file-order pass
    std::vector<char> early(nt, 0);
    for (const sti::Output& o : ix.outputs) {
        const uint64_t wend = ix.tensors[o.tensor].end;
        for (int64_t s : {o.scale, o.scale2})
            if (s >= 0 && ix.tensors[size_t(s)].end > wend + p.chunk_bytes) early[size_t(s)] = 1;
    }
    std::vector<uint32_t> by_offset(nt);
    std::iota(by_offset.begin(), by_offset.end(), 0u);
    std::sort(by_offset.begin(), by_offset.end(), [&](uint32_t a, uint32_t b) {
        return ix.tensors[a].begin != ix.tensors[b].begin ? ix.tensors[a].begin < ix.tensors[b].begin : a < b;
    });
    int64_t fill = -1;
    for (int pass = 0; pass < 2; ++pass) {  // early tensors, then everything else in file order
        if (pass == 1) fill = fill < 0 ? -1 : int64_t(p.chunk_bytes);  // the file-order pass starts a new step
        for (uint32_t t : by_offset)
            if (bool(early[t]) == (pass == 0)) add_bytes(p, ix.tensors[t].begin, ix.tensors[t].end, fill);
    }
    if (p.steps.empty()) p.steps.push_back(st_stream_step{});  // nothing to read: one empty step

    // the step that copies each tensor's last byte (the ranges tile the data section)
    std::vector<st_stream_range> sorted(p.ranges);
    std::sort(sorted.begin(), sorted.end(), [](const st_stream_range& a, const st_stream_range& b) { return a.begin < b.begin; });
    std::vector<uint32_t> done(nt, 0);
    for (size_t t = 0; t < nt; ++t) {
        const sti::Tensor& x = ix.tensors[t];
        if (x.end == x.begin) continue;  // no bytes: ready at step 0
        auto it = std::upper_bound(sorted.begin(), sorted.end(), x.end - 1,
                                   [](uint64_t v, const st_stream_range& r) { return v < r.begin; });
        done[t] = std::prev(it)->step;
    }
    std::vector<uint32_t> ready(no);
    for (size_t k = 0; k < no; ++k) {
        const sti::Output& o = ix.outputs[k];
        uint32_t s = done[o.tensor];
        if (o.scale >= 0) s = std::max(s, done[size_t(o.scale)]);
        if (o.scale2 >= 0) s = std::max(s, done[size_t(o.scale2)]);
        ready[k] = s;
    }
    p.order.resize(no);
    std::iota(p.order.begin(), p.order.end(), 0u);
    std::stable_sort(p.order.begin(), p.order.end(), [&](uint32_t a, uint32_t b) { return ready[a] < ready[b]; });
    size_t k = 0;
    for (uint32_t s = 0; s < p.steps.size(); ++s) {
        st_stream_step& st = p.steps[s];
        st.first_out = uint32_t(k);
        while (k < no && ready[p.order[k]] == s) ++k;
        st.n_out = uint32_t(k - st.first_out);
        st.table_offset = p.tables.size();
        st.units = 0;
        if (st.n_out) {
            std::vector<unsigned char> t = sti::build_table(ix, p.order.data() + st.first_out, st.n_out, &st.units);
            p.tables.insert(p.tables.end(), t.begin(), t.end());
            p.tables.resize((p.tables.size() + 63) / 64 * 64, 0);
        }
    }
}

}  // namespace

extern "C" st_status st_stream_plan_build(const st_index* idx, uint64_t chunk_bytes, st_stream_plan** out) {
    sti::clear_error();
    if (!idx || !out) return st_fail(ST_E_ARG, "st_stream_plan_build: null pointer");
    *out = nullptr;
    if (chunk_bytes < kMinChunk)
        return st_fail(ST_E_ARG, "st_stream_plan_build: chunk of %llu bytes, at least %llu needed",
                       (unsigned long long)chunk_bytes, (unsigned long long)kMinChunk);
    if (idx->outputs.size() >= (uint64_t(1) << 32)) return st_fail(ST_E_SHAPE, "more than 2^32 outputs");
    st_stream_plan* p = nullptr;
    try {
        p = new st_stream_plan;
        p->owner = idx;
        p->chunk_bytes = chunk_bytes;
        build(*idx, *p);
        if (p->steps.size() >= (uint64_t(1) << 32) || p->ranges.size() >= (uint64_t(1) << 32))
            throw std::length_error("too many steps");
    } catch (const std::bad_alloc&) {
        delete p;
        return st_fail(ST_E_NOMEM, "out of host memory");
    } catch (const std::length_error&) {
        delete p;
        return st_fail(ST_E_SHAPE, "st_stream_plan_build: a step needs 2^32 or more work units, or too many steps");
    }
    *out = p;
    return ST_OK;
}

extern "C" void st_stream_plan_free(st_stream_plan* plan) { delete plan; }

bool st_stream_plan_of(const st_stream_plan* plan, const st_index* idx) { return plan && plan->owner == idx; }

extern "C" uint64_t st_stream_plan_chunk_bytes(const st_stream_plan* plan) { return plan ? plan->chunk_bytes : 0; }

extern "C" size_t st_stream_plan_num_steps(const st_stream_plan* plan) { return plan ? plan->steps.size() : 0; }

extern "C" st_status st_stream_plan_step(const st_stream_plan* plan, size_t s, st_stream_step* out) {
    if (!plan || !out) return st_fail(ST_E_ARG, "st_stream_plan_step: null pointer");
    if (s >= plan->steps.size())
        return st_fail(ST_E_ARG, "st_stream_plan_step: step %zu of %zu", s, plan->steps.size());
    *out = plan->steps[s];
    return ST_OK;
}

extern "C" const st_stream_range* st_stream_plan_ranges(const st_stream_plan* plan, size_t* n) {
    if (n) *n = plan ? plan->ranges.size() : 0;
    return plan ? plan->ranges.data() : nullptr;
}

extern "C" const uint32_t* st_stream_plan_order(const st_stream_plan* plan, size_t* n) {
    if (n) *n = plan ? plan->order.size() : 0;
    return plan ? plan->order.data() : nullptr;
}

extern "C" const void* st_stream_plan_tables(const st_stream_plan* plan, size_t* bytes) {
    if (bytes) *bytes = plan ? plan->tables.size() : 0;
    return plan ? plan->tables.data() : nullptr;
}
