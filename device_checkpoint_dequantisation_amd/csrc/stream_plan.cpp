// Streaming plans: staging steps over a checkpoint's bytes and the outputs each step completes.
//
// The pages' disk tier reads only the byte ranges a load needs into pinned host memory, copies them
// to the GPU and releases the host buffer; a state dict loads tensors on demand and a RAM tier keeps
// recently read weights ("Disk tier safetensors streaming design audit", "Strategy summary / Range
// reads and tiering" and "Disk tier integration").  A plan covers either every output or a chosen
// set of outputs:
//  * The bytes it reads are the weight and scale tensors of those outputs (the whole data section
//    for a whole-file plan), as runs of file-adjacent tensors (gaps up to kMergeGap are read too).
//  * Where they go: at their data-section offsets in a blob of st_index_blob_bytes, or, packed,
//    into a compact blob holding only those runs, each run starting on a 256-byte boundary plus its
//    data-section offset mod 256, so the kernel sees the same alignment as in the full blob.
//  * Steps: the runs are cut into steps of at most chunk_bytes, in file order, except that a scale
//    tensor lying more than one chunk past the end of its weight (a checkpoint that stores all
//    scales at the end, say) is staged first, packed into the leading steps.
//  * Each output is attached to the first step after which every byte of its inputs has been
//    copied, and each step carries a work table for just those outputs.
// st_stream_file (stage.cpp) executes a plan; st_read_plan reads its bytes into host memory.
#include <algorithm>
#include <new>
#include <numeric>
#include <stdexcept>
#include <vector>

#include "index_impl.h"

struct st_stream_plan {
    const st_index* owner = nullptr;       // the index it was planned from
    uint64_t chunk_bytes = 0;
    uint64_t blob_bytes = 0;               // device blob the tables address
    uint32_t flags = 0;
    std::vector<st_stream_range> ranges;   // step-major
    std::vector<st_stream_step> steps;
    std::vector<uint32_t> order;           // output indices, step-major
    std::vector<unsigned char> tables;     // every step's work table, each 64-byte aligned
};

namespace {

constexpr uint64_t kMinChunk = uint64_t(64) << 10;
constexpr uint64_t kMergeGap = 4096;  // unneeded bytes read to join two runs

struct Run {
    uint64_t begin, end, dst;
    bool early;
};

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Appends the bytes [b, e) of a run, destined for blob offset dst, opening a new step whenever the
// current one is full.  `fill` is the byte count of the open step (-1: none open).
void add_bytes(st_stream_plan& p, uint64_t b, uint64_t e, uint64_t dst, int64_t& fill) {
    while (b < e) {
        if (fill < 0 || uint64_t(fill) == p.chunk_bytes) {
            st_stream_step s{};
            s.first_range = uint32_t(p.ranges.size());
            p.steps.push_back(s);
            fill = 0;
        }
        const uint64_t take = std::min<uint64_t>(e - b, p.chunk_bytes - uint64_t(fill));
        st_stream_step& s = p.steps.back();
        if (s.n_ranges && p.ranges.back().end == b && p.ranges.back().dst + (b - p.ranges.back().begin) == dst) {
            p.ranges.back().end += take;  // contiguous with the step's previous range, in file and blob
        } else {
            p.ranges.push_back(st_stream_range{b, b + take, dst, uint32_t(p.steps.size() - 1), 0});
            ++s.n_ranges;
        }
        s.bytes += take;
        fill += int64_t(take);
        b += take;
        dst += take;
    }
}

void build(const st_index& ix, const std::vector<uint32_t>& sel, bool pack, st_stream_plan& p) {
    const size_t nt = ix.tensors.size();
    // the tensors the selected outputs read, and which of them are staged early
    std::vector<char> need(nt, 0), early(nt, 0);
    for (uint32_t k : sel) {
        const sti::Output& o = ix.outputs[k];
        need[o.tensor] = 1;
        const uint64_t wend = ix.tensors[o.tensor].end;
        for (int64_t s : {o.scale, o.scale2})
            if (s >= 0) {
                need[size_t(s)] = 1;
                if (ix.tensors[size_t(s)].end > wend + p.chunk_bytes) early[size_t(s)] = 1;
            }
    }
    std::vector<uint32_t> by_offset;
    for (uint32_t t = 0; t < nt; ++t)
        if (need[t] && ix.tensors[t].end > ix.tensors[t].begin) by_offset.push_back(t);
    std::sort(by_offset.begin(), by_offset.end(), [&](uint32_t a, uint32_t b) {
        return ix.tensors[a].begin != ix.tensors[b].begin ? ix.tensors[a].begin < ix.tensors[b].begin : a < b;
    });
    // runs of file-adjacent tensors, early ones separately; a gap bridged by a run never holds
    // bytes of the other pass (they would be read twice)
    std::vector<uint64_t> early_begin, late_begin;
    for (uint32_t t : by_offset) (early[t] ? early_begin : late_begin).push_back(ix.tensors[t].begin);
    auto none_in = [](const std::vector<uint64_t>& v, uint64_t b, uint64_t e) {  // no element in [b, e)
        auto it = std::lower_bound(v.begin(), v.end(), b);
        return it == v.end() || *it >= e;
    };
    std::vector<Run> runs;
    for (int pass = 0; pass < 2; ++pass)
        for (uint32_t t : by_offset) {
            if (bool(early[t]) != (pass == 0)) continue;
            const sti::Tensor& x = ix.tensors[t];
            const std::vector<uint64_t>& other = pass == 0 ? late_begin : early_begin;
            if (!runs.empty() && runs.back().early == (pass == 0) && x.begin >= runs.back().end &&
                x.begin - runs.back().end <= kMergeGap && none_in(other, runs.back().end, x.begin))
                runs.back().end = std::max(runs.back().end, x.end);
            else
                runs.push_back(Run{x.begin, x.end, 0, pass == 0});
        }
    // destinations
    uint64_t cursor = 0;
    for (Run& r : runs) {
        if (pack) {
            r.dst = round_up(cursor, 256) + r.begin % 256;
            cursor = r.dst + (r.end - r.begin);
        } else {
            r.dst = r.begin;
        }
    }
    p.blob_bytes = pack ? round_up(cursor + 64, 256) : round_up(ix.data_size + 64, 256);
    int64_t fill = -1;
    bool in_early = true;
    for (const Run& r : runs) {
        if (in_early && !r.early) {
            in_early = false;
            if (fill >= 0) fill = int64_t(p.chunk_bytes);  // the file-order pass starts a new step
        }
        add_bytes(p, r.begin, r.end, r.dst, fill);
    }
    if (p.steps.empty()) p.steps.push_back(st_stream_step{});  // nothing to read: one empty step

    // where each needed tensor lands, and the step that copies its last byte
    std::vector<st_stream_range> sorted(p.ranges);
    std::sort(sorted.begin(), sorted.end(),
              [](const st_stream_range& a, const st_stream_range& b) { return a.begin < b.begin; });
    auto range_of = [&](uint64_t byte) {
        return std::prev(std::upper_bound(sorted.begin(), sorted.end(), byte,
                                          [](uint64_t v, const st_stream_range& r) { return v < r.begin; }));
    };
    std::vector<uint32_t> done(nt, 0);
    std::vector<uint64_t> at(nt, 0);
    for (uint32_t t : by_offset) {
        const sti::Tensor& x = ix.tensors[t];
        auto first = range_of(x.begin);
        at[t] = first->dst + (x.begin - first->begin);
        done[t] = range_of(x.end - 1)->step;
    }
    std::vector<uint32_t> ready(ix.outputs.size(), 0);
    for (uint32_t k : sel) {
        const sti::Output& o = ix.outputs[k];
        uint32_t s = done[o.tensor];
        if (o.scale >= 0) s = std::max(s, done[size_t(o.scale)]);
        if (o.scale2 >= 0) s = std::max(s, done[size_t(o.scale2)]);
        ready[k] = s;
    }
    p.order = sel;
    std::stable_sort(p.order.begin(), p.order.end(), [&](uint32_t a, uint32_t b) { return ready[a] < ready[b]; });
    size_t k = 0;
    const uint64_t* where = pack ? at.data() : nullptr;
    for (uint32_t s = 0; s < p.steps.size(); ++s) {
        st_stream_step& st = p.steps[s];
        st.first_out = uint32_t(k);
        while (k < p.order.size() && ready[p.order[k]] == s) ++k;
        st.n_out = uint32_t(k - st.first_out);
        st.table_offset = p.tables.size();
        st.units = 0;
        if (st.n_out) {
            std::vector<unsigned char> t = sti::build_table(ix, p.order.data() + st.first_out, st.n_out, &st.units, where);
            p.tables.insert(p.tables.end(), t.begin(), t.end());
            p.tables.resize((p.tables.size() + 63) / 64 * 64, 0);
        }
    }
}

st_status make_plan(const st_index* idx, const uint32_t* sel, size_t k, bool all, uint64_t chunk_bytes, uint32_t flags,
                    st_stream_plan** out) {
    sti::clear_error();
    if (!idx || !out || (!all && k && !sel)) return st_fail(ST_E_ARG, "st_stream_plan: null pointer");
    *out = nullptr;
    if (chunk_bytes < kMinChunk)
        return st_fail(ST_E_ARG, "st_stream_plan: chunk of %llu bytes, at least %llu needed",
                       (unsigned long long)chunk_bytes, (unsigned long long)kMinChunk);
    if (flags & ~uint32_t(ST_PLAN_PACK)) return st_fail(ST_E_ARG, "st_stream_plan: unknown flags 0x%x", flags);
    const size_t n_out = idx->outputs.size();
    if (n_out >= (uint64_t(1) << 32)) return st_fail(ST_E_SHAPE, "more than 2^32 outputs");
    std::vector<uint32_t> chosen;
    st_stream_plan* p = nullptr;
    try {
        if (all) {
            chosen.resize(n_out);
            std::iota(chosen.begin(), chosen.end(), 0u);
        } else {
            std::vector<char> seen(n_out, 0);
            for (size_t j = 0; j < k; ++j) {
                if (sel[j] >= n_out)
                    return st_fail(ST_E_ARG, "st_stream_plan_select: output %u out of range (%zu)", sel[j], n_out);
                if (seen[sel[j]]) return st_fail(ST_E_ARG, "st_stream_plan_select: output %u selected twice", sel[j]);
                seen[sel[j]] = 1;
                chosen.push_back(sel[j]);
            }
        }
        p = new st_stream_plan;
        p->owner = idx;
        p->chunk_bytes = chunk_bytes;
        p->flags = flags;
        build(*idx, chosen, (flags & ST_PLAN_PACK) != 0, *p);
        if (p->steps.size() >= (uint64_t(1) << 32) || p->ranges.size() >= (uint64_t(1) << 32))
            throw std::length_error("too many steps");
    } catch (const std::bad_alloc&) {
        delete p;
        return st_fail(ST_E_NOMEM, "out of host memory");
    } catch (const std::length_error& e) {
        delete p;
        return st_fail(ST_E_SHAPE, "st_stream_plan: %s", e.what());
    }
    *out = p;
    return ST_OK;
}

}  // namespace

extern "C" st_status st_stream_plan_build(const st_index* idx, uint64_t chunk_bytes, st_stream_plan** out) {
    return make_plan(idx, nullptr, 0, true, chunk_bytes, 0, out);
}

extern "C" st_status st_stream_plan_select(const st_index* idx, const uint32_t* sel, size_t k, uint64_t chunk_bytes,
                                           uint32_t flags, st_stream_plan** out) {
    return make_plan(idx, sel, k, false, chunk_bytes, flags, out);
}

extern "C" void st_stream_plan_free(st_stream_plan* plan) { delete plan; }

bool st_stream_plan_of(const st_stream_plan* plan, const st_index* idx) { return plan && plan->owner == idx; }

extern "C" uint64_t st_stream_plan_chunk_bytes(const st_stream_plan* plan) { return plan ? plan->chunk_bytes : 0; }

extern "C" uint64_t st_stream_plan_blob_bytes(const st_stream_plan* plan) { return plan ? plan->blob_bytes : 0; }

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
