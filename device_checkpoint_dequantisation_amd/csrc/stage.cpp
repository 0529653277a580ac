// Staging: the file's data section -> pinned host ring -> one device blob.
//
// The pages ("Disk tier safetensors streaming design audit", "Strategy summary / Range reads
// and tiering") read only a tensor's byte range into (optionally pinned) host memory, copy it
// to the GPU and release the host buffer.  Byte ranges are read by a few threads into a ring
// carved from the caller's pinned buffer, and each slot is copied with hipMemcpyAsync on a side
// stream while the next one is being read.  An event per ring slot keeps a slot from being
// overwritten before its copy has finished, and an event per caller buffer keeps the next call
// from reading into a ring that the previous call's copies are still reading.
//  * st_stage_file: the whole data section, in slot-sized chunks.
//  * st_stream_file: the steps of a stream plan; after each step's copies the compute stream waits
//    for them and decodes the outputs the step completes, so decoding overlaps later reads and
//    copies.
//  * st_read_plan: a plan's ranges straight into host memory (the RAM tier), no GPU calls.
#include <fcntl.h>
#include <sys/stat.h>
#include <sys/uio.h>
#include <unistd.h>

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cerrno>
#include <chrono>
#include <condition_variable>
#include <cstring>
#include <memory>
#include <mutex>
#include <thread>
#include <vector>

#include "index_impl.h"
#include "st_internal.h"

namespace {

constexpr size_t kMinPinned = size_t(2) << 20;
constexpr int kSlots = 4;
#ifndef ST_READERS
#define ST_READERS 8
#endif
constexpr int kReaders = ST_READERS;  // pool threads; the calling thread reads too

struct Piece {
    char* dst;
    uint64_t off;  // file offset
    size_t len;
};

// Reader threads.  read() splits a batch of ranges of one file into pieces and reads them with
// pread on the pool's threads and the calling thread; every thread takes part in every batch, so
// a batch is over once all of them have checked in.  One pool serves the whole process (see
// Readers below): starting eight threads per call cost a 113 MB per-layer load about 0.1 ms
// (measured on an MI355X host, 2.72-2.82 ms per layer against 2.66).
class ReaderPool {
  public:
    ReaderPool() {
        for (int i = 0; i < kReaders; ++i) threads_.emplace_back([this] { worker(); });
    }
    ~ReaderPool() {
        {
            std::lock_guard<std::mutex> lk(m_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : threads_) t.join();
    }
    // False if a read failed or hit the end of the file.  Pieces: ranges whose pages are in the page
    // cache are memory copies, which the threads share best in pieces of about a (2 * readers)-th of
    // the batch; ranges still on disk are read in pieces of kColdPiece, since the kernel submits a
    // read's missing pages together and larger reads keep more of the disk's queue busy (measured
    // on MI355X hosts, cold 128 MiB batches: 3.3 GB/s in 7 MiB pieces, 6.8 in 32 MiB, 7.3 in 64 MiB).
    bool read(int fd, const std::vector<Piece>& ranges) {
        size_t total = 0;
        for (const Piece& r : ranges) total += r.len;
        const size_t piece = in_page_cache(fd, ranges)
                                 ? std::max<size_t>(size_t(1) << 20, (total / (2 * (kReaders + 1)) + 4095) & ~size_t(4095))
                                 : kColdPiece;
        std::vector<Piece> pieces;
        for (const Piece& r : ranges)
            for (size_t b = 0; b < r.len; b += piece)
                pieces.push_back(Piece{r.dst + b, r.off + b, std::min(piece, r.len - b)});
        {
            std::lock_guard<std::mutex> lk(m_);
            fd_ = fd;
            pieces_.swap(pieces);
            next_.store(0);
            ok_.store(true);
            checked_in_ = 0;
            ++gen_;
        }
        cv_.notify_all();
        drain();
        std::unique_lock<std::mutex> lk(m_);
        done_cv_.wait(lk, [this] { return checked_in_ == threads_.size(); });
        return ok_.load();
    }

  private:
    static constexpr size_t kColdPiece = size_t(64) << 20;
    // Whether the first, middle and last byte of the batch's ranges (the first 16 of them) are in
    // the page cache: a one-byte preadv2 with RWF_NOWAIT returns EAGAIN instead of waiting for the
    // disk.  Any other failure (a kernel without RWF_NOWAIT for buffered reads) counts as cached,
    // which keeps the smaller pieces; the reads themselves report real errors.
    static bool in_page_cache(int fd, const std::vector<Piece>& ranges) {
        size_t probed = 0;
        for (const Piece& r : ranges) {
            if (r.len == 0) continue;
            const uint64_t at[3] = {r.off, r.off + r.len / 2, r.off + r.len - 1};
            for (uint64_t o : at) {
                char b;
                struct iovec v = {&b, 1};
                if (preadv2(fd, &v, 1, off_t(o), RWF_NOWAIT) < 0 && errno == EAGAIN) return false;
            }
            if (++probed == 16) break;
        }
        return true;
    }
    void drain() {
        for (size_t i = next_.fetch_add(1); i < pieces_.size(); i = next_.fetch_add(1)) {
            const Piece& p = pieces_[i];
            size_t b = 0;
            while (b < p.len) {
                const ssize_t r = pread(fd_, p.dst + b, p.len - b, off_t(p.off + b));
                if (r < 0 && errno == EINTR) continue;  // interrupted before any byte was read
                if (r <= 0) {
                    ok_.store(false);
                    break;
                }
                b += size_t(r);
            }
        }
    }
    void worker() {
        uint64_t seen = 0;
        std::unique_lock<std::mutex> lk(m_);
        for (;;) {
            cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
            if (stop_) return;
            seen = gen_;
            lk.unlock();
            drain();
            lk.lock();
            if (++checked_in_ == threads_.size()) done_cv_.notify_all();
        }
    }

    int fd_ = -1;                 // the batch's file; written only while every thread is idle
    std::vector<std::thread> threads_;
    std::mutex m_;
    std::condition_variable cv_, done_cv_;
    std::vector<Piece> pieces_;   // written only while every thread is idle
    std::atomic<size_t> next_{0};
    std::atomic<bool> ok_{true};
    size_t checked_in_ = 0;
    uint64_t gen_ = 0;
    bool stop_ = false;
};

// The process's reader pool, taken for the length of one call.  A call that finds it in use (a
// concurrent call from another thread) gets a pool of its own for that call.  The shared pool is
// never destroyed (its threads wait on a condition variable until the process ends), and a child
// process created by fork() starts a pool of its own, since the parent's threads do not exist in it.
class Readers {
  public:
    Readers() {
        std::unique_lock<std::mutex> lk(shared_mutex(), std::try_to_lock);
        if (lk.owns_lock()) {
            static ReaderPool* pool = nullptr;
            static pid_t owner = 0;
            if (!pool || owner != getpid()) {
                pool = new ReaderPool();  // any pool left from before a fork is abandoned
                owner = getpid();
            }
            lock_ = std::move(lk);
            pool_ = pool;
        } else {
            own_.reset(new ReaderPool());
            pool_ = own_.get();
        }
    }
    bool read(int fd, const std::vector<Piece>& ranges) { return pool_->read(fd, ranges); }

  private:
    static std::mutex& shared_mutex() {
        static std::mutex m;
        return m;
    }
    std::unique_lock<std::mutex> lock_;
    std::unique_ptr<ReaderPool> own_;
    ReaderPool* pool_ = nullptr;
};

// An open file descriptor, closed on scope exit.
struct FileFd {
    int fd = -1;
    ~FileFd() {
        if (fd >= 0) close(fd);
    }
};

// Opens `path` and checks that its size is what the index expects.
st_status open_checked(const char* path, const st_index* idx, FileFd& f) {
    const uint64_t want = st_index_data_offset(idx) + st_index_data_size(idx);
    f.fd = open(path, O_RDONLY | O_CLOEXEC);
    if (f.fd < 0) return st_fail(ST_E_IO, "cannot open %s", path);
    struct stat sb;
    if (fstat(f.fd, &sb) != 0 || uint64_t(sb.st_size) != want)
        return st_fail(ST_E_IO, "%s is %lld bytes, the index expects %llu", path, (long long)sb.st_size,
                       (unsigned long long)want);
    return ST_OK;
}

struct RingEvents {
    hipEvent_t ev[kSlots];
    int n = 0;
    st_status create() {
        for (; n < kSlots; ++n)
            if (hipEventCreateWithFlags(&ev[n], hipEventDisableTiming) != hipSuccess)
                return st_fail(ST_E_HIP, "hipEventCreate failed");
        return ST_OK;
    }
    ~RingEvents() {
        for (int k = 0; k < n; ++k) (void)hipEventDestroy(ev[k]);
    }
};

// Copies still reading a caller's pinned buffer when a call returns.  st_stage_file and
// st_stream_file return once their copies are enqueued, so the side stream may still be reading
// the ring; a later call handed the same buffer must not read the file into it before then.  Each
// call records an event on its side stream after its last copy and files it under the buffer's
// address range; the next call whose buffer overlaps that range waits for the event on the host
// before its first read.  Entries are few (one per ring a process uses); past kMaxEntries the
// oldest is waited for and dropped.
class PinnedInFlight {
  public:
    static PinnedInFlight& get() {
        static PinnedInFlight* p = new PinnedInFlight();  // never destroyed: events outlive static teardown
        return *p;
    }
    // Waits for every recorded copy out of [base, base + bytes).
    st_status wait(const void* base, size_t bytes, const char* who) {
        std::vector<hipEvent_t> evs;
        {
            std::lock_guard<std::mutex> lk(m_);
            for (size_t i = 0; i < v_.size();) {
                if (overlaps(v_[i], base, bytes)) {
                    evs.push_back(v_[i].ev);
                    v_.erase(v_.begin() + long(i));
                } else {
                    ++i;
                }
            }
        }
        st_status r = ST_OK;
        for (hipEvent_t e : evs) {
            if (hipEventSynchronize(e) != hipSuccess && r == ST_OK)
                r = st_fail(ST_E_HIP, "%s: waiting for an earlier call's copies out of the pinned buffer failed", who);
            (void)hipEventDestroy(e);
        }
        return r;
    }
    // Records the point after the last copy out of [base, base + bytes) on `side`; if no event can
    // be recorded there, waits for the stream instead.
    void record(const void* base, size_t bytes, hipStream_t side) {
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
            (void)hipStreamSynchronize(side);
            return;
        }
        if (hipEventRecord(e, side) != hipSuccess) {
            (void)hipEventDestroy(e);
            (void)hipStreamSynchronize(side);
            return;
        }
        hipEvent_t oldest = nullptr;
        {
            std::lock_guard<std::mutex> lk(m_);
            v_.push_back(Entry{static_cast<const char*>(base), bytes, e});
            if (v_.size() > kMaxEntries) {
                oldest = v_.front().ev;
                v_.erase(v_.begin());
            }
        }
        if (oldest) {
            (void)hipEventSynchronize(oldest);
            (void)hipEventDestroy(oldest);
        }
    }

  private:
    struct Entry {
        const char* base;
        size_t bytes;
        hipEvent_t ev;
    };
    static bool overlaps(const Entry& x, const void* base, size_t bytes) {
        const char* b = static_cast<const char*>(base);
        return x.base < b + bytes && b < x.base + x.bytes;
    }
    static constexpr size_t kMaxEntries = 64;
    std::mutex m_;
    std::vector<Entry> v_;
};

double seconds_since(std::chrono::steady_clock::time_point t0) {
    return std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
}

}  // namespace

extern "C" st_status st_stage_file(const char* path, const st_index* idx, void* blob_dev, void* pinned,
                                   size_t pinned_bytes, void* side_stream, void* done_event, double* seconds_read) {
    if (seconds_read) *seconds_read = 0;
    if (!path || !idx || !blob_dev || !pinned) return st_fail(ST_E_ARG, "st_stage_file: null pointer");
    if (pinned_bytes < kMinPinned)
        return st_fail(ST_E_ARG, "st_stage_file: pinned buffer of %zu bytes, at least %zu needed", pinned_bytes, kMinPinned);
    if (reinterpret_cast<uintptr_t>(blob_dev) % ST_BLOB_ALIGN)
        return st_fail(ST_E_ARG, "st_stage_file: blob is not %d-byte aligned", ST_BLOB_ALIGN);
    const uint64_t off0 = st_index_data_offset(idx), size = st_index_data_size(idx);
    FileFd file;
    st_status status = open_checked(path, idx, file);
    if (status != ST_OK) return status;
    if ((status = PinnedInFlight::get().wait(pinned, pinned_bytes, "st_stage_file")) != ST_OK) return status;
    RingEvents ring;
    if ((status = ring.create()) != ST_OK) return status;
    Readers pool;
    hipStream_t stream = static_cast<hipStream_t>(side_stream);
    const size_t chunk = (pinned_bytes / kSlots) & ~size_t(4095);
    double t_read = 0;
    uint64_t done = 0;
    for (uint64_t i = 0; done < size; ++i) {
        const int s = int(i % kSlots);
        char* slot = static_cast<char*>(pinned) + size_t(s) * chunk;
        const size_t len = size_t(std::min<uint64_t>(chunk, size - done));
        if (i >= kSlots && hipEventSynchronize(ring.ev[s]) != hipSuccess) {
            status = st_fail(ST_E_HIP, "st_stage_file: waiting for a staging copy failed");
            break;
        }
        auto t0 = std::chrono::steady_clock::now();
        const bool ok = pool.read(file.fd, {Piece{slot, off0 + done, len}});
        t_read += seconds_since(t0);
        if (!ok) {
            status = st_fail(ST_E_IO, "read of %s failed at byte %llu", path, (unsigned long long)(off0 + done));
            break;
        }
        if (hipMemcpyAsync(static_cast<char*>(blob_dev) + done, slot, len, hipMemcpyHostToDevice, stream) != hipSuccess ||
            hipEventRecord(ring.ev[s], stream) != hipSuccess) {
            status = st_fail(ST_E_HIP, "st_stage_file: hipMemcpyAsync of %zu bytes failed", len);
            break;
        }
        done += len;
    }
    if (status == ST_OK && done_event && hipEventRecord(static_cast<hipEvent_t>(done_event), stream) != hipSuccess)
        status = st_fail(ST_E_HIP, "st_stage_file: hipEventRecord failed");
    if (status != ST_OK) (void)hipStreamSynchronize(stream);  // nothing may still read the ring
    else PinnedInFlight::get().record(pinned, pinned_bytes, stream);
    if (seconds_read) *seconds_read = t_read;
    return status;
}

extern "C" st_status st_stream_file(const char* path, const st_index* idx, const st_stream_plan* plan, void* blob_dev,
                                    const void* tables_dev, void* const* outs_dev, void* pinned, size_t pinned_bytes,
                                    void* side_stream, void* compute_stream, void* done_event, st_stream_stats* stats) {
    if (stats) *stats = st_stream_stats{};
    if (!path || !idx || !plan || !blob_dev || !pinned) return st_fail(ST_E_ARG, "st_stream_file: null pointer");
    if (!st_stream_plan_of(plan, idx)) return st_fail(ST_E_ARG, "st_stream_file: the plan was built from another index");
    const uint64_t chunk = st_stream_plan_chunk_bytes(plan);
    if (pinned_bytes / kSlots < chunk)
        return st_fail(ST_E_ARG, "st_stream_file: pinned buffer of %zu bytes, %d chunks of %llu bytes needed", pinned_bytes,
                       kSlots, (unsigned long long)chunk);
    if (reinterpret_cast<uintptr_t>(blob_dev) % ST_BLOB_ALIGN)
        return st_fail(ST_E_ARG, "st_stream_file: blob is not %d-byte aligned", ST_BLOB_ALIGN);
    size_t table_bytes = 0, n_order = 0, n_ranges = 0;
    const unsigned char* tables_host = static_cast<const unsigned char*>(st_stream_plan_tables(plan, &table_bytes));
    (void)st_stream_plan_order(plan, &n_order);
    const st_stream_range* ranges = st_stream_plan_ranges(plan, &n_ranges);
    if (table_bytes && (!tables_dev || reinterpret_cast<uintptr_t>(tables_dev) % 64))
        return st_fail(ST_E_ARG, "st_stream_file: tables_dev is null or not 64-byte aligned");
    if (n_order && !outs_dev) return st_fail(ST_E_ARG, "st_stream_file: outs_dev is null");

    const uint64_t off0 = st_index_data_offset(idx);
    FileFd file;
    st_status status = open_checked(path, idx, file);
    if (status != ST_OK) return status;
    if ((status = PinnedInFlight::get().wait(pinned, pinned_bytes, "st_stream_file")) != ST_OK) return status;
    RingEvents ring;
    if ((status = ring.create()) != ST_OK) return status;
    Readers pool;
    std::vector<Piece> batch;
    hipStream_t side = static_cast<hipStream_t>(side_stream), compute = static_cast<hipStream_t>(compute_stream);
    st_stream_stats st{};
    st.seconds_first_launch = -1;
    const auto t_call = std::chrono::steady_clock::now();
    int last_slot = -1;  // ring slot of the last step that copied bytes
    const size_t nsteps = st_stream_plan_num_steps(plan);
    for (size_t s = 0; status == ST_OK && s < nsteps; ++s) {
        st_stream_step step;
        (void)st_stream_plan_step(plan, s, &step);
        const int slot_id = int(s % kSlots);
        char* slot = static_cast<char*>(pinned) + size_t(slot_id) * chunk;
        if (step.bytes) {
            if (s >= size_t(kSlots)) {
                auto t0 = std::chrono::steady_clock::now();
                if (hipEventSynchronize(ring.ev[slot_id]) != hipSuccess) {
                    status = st_fail(ST_E_HIP, "st_stream_file: waiting for a staging copy failed");
                    break;
                }
                st.seconds_wait += seconds_since(t0);
            }
            size_t pos = 0;
            batch.clear();
            for (uint32_t r = step.first_range; r < step.first_range + step.n_ranges && r < n_ranges; ++r) {
                const size_t len = size_t(ranges[r].end - ranges[r].begin);
                batch.push_back(Piece{slot + pos, off0 + ranges[r].begin, len});
                pos += len;
            }
            auto t0 = std::chrono::steady_clock::now();
            if (!pool.read(file.fd, batch))
                status = st_fail(ST_E_IO, "read of %s failed in step %zu", path, s);
            st.seconds_read += seconds_since(t0);
            if (status != ST_OK) break;
            pos = 0;
            for (uint32_t r = step.first_range; r < step.first_range + step.n_ranges && r < n_ranges; ++r) {
                const size_t len = size_t(ranges[r].end - ranges[r].begin);
                if (hipMemcpyAsync(static_cast<char*>(blob_dev) + ranges[r].dst, slot + pos, len, hipMemcpyHostToDevice,
                                   side) != hipSuccess) {
                    status = st_fail(ST_E_HIP, "st_stream_file: hipMemcpyAsync of %zu bytes failed", len);
                    break;
                }
                pos += len;
            }
            if (status != ST_OK) break;
            if (hipEventRecord(ring.ev[slot_id], side) != hipSuccess) {
                status = st_fail(ST_E_HIP, "st_stream_file: hipEventRecord failed");
                break;
            }
            st.bytes_read += pos;
            ++st.steps;
            last_slot = slot_id;
        }
        if (step.units) {
            // The side stream runs its copies in order, so the event of the last step that copied
            // anything covers every byte this step's outputs read (a plan attaches an output to a
            // step that copies its last byte, so that is normally this step's own event).
            if (last_slot >= 0 && hipStreamWaitEvent(compute, ring.ev[last_slot], 0) != hipSuccess) {
                status = st_fail(ST_E_HIP, "st_stream_file: hipStreamWaitEvent failed");
                break;
            }
            st_table_header h;  // the step table's store policy, from the plan's host copy
            memcpy(&h, tables_host + step.table_offset, sizeof h);
            status = st_materialize_as(blob_dev, static_cast<const char*>(tables_dev) + step.table_offset,
                                       size_t(step.units), outs_dev + step.first_out, st_index_out_dtype(idx),
                                       (h.flags & ST_TABLE_STREAM_STORES) ? ST_MAT_STREAM_STORES : 0u, compute_stream);
            if (status != ST_OK) break;
            if (st.launches++ == 0) st.seconds_first_launch = seconds_since(t_call);
        }
    }
    if (status == ST_OK && done_event && hipEventRecord(static_cast<hipEvent_t>(done_event), compute) != hipSuccess)
        status = st_fail(ST_E_HIP, "st_stream_file: hipEventRecord failed");
    if (status != ST_OK) (void)hipStreamSynchronize(side);  // nothing may still read the ring
    else PinnedInFlight::get().record(pinned, pinned_bytes, side);
    if (stats) *stats = st;
    return status;
}

extern "C" st_status st_read_plans(const char* path, const st_index* idx, const st_stream_plan* const* plans,
                                   void* const* host_blobs, const size_t* host_bytes, size_t n, double* seconds_read) {
    if (seconds_read) *seconds_read = 0;
    if (!path || !idx || (n && (!plans || !host_blobs || !host_bytes))) return st_fail(ST_E_ARG, "st_read_plans: null pointer");
    std::vector<Piece> batch;
    const uint64_t off0 = st_index_data_offset(idx);
    for (size_t j = 0; j < n; ++j) {
        if (!plans[j] || !host_blobs[j]) return st_fail(ST_E_ARG, "st_read_plans: null plan or buffer %zu", j);
        if (!st_stream_plan_of(plans[j], idx))
            return st_fail(ST_E_ARG, "st_read_plans: plan %zu was built from another index", j);
        if (host_bytes[j] < st_stream_plan_blob_bytes(plans[j]))
            return st_fail(ST_E_ARG, "st_read_plans: host buffer %zu holds %zu bytes, %llu needed", j, host_bytes[j],
                           (unsigned long long)st_stream_plan_blob_bytes(plans[j]));
        size_t nr = 0;
        const st_stream_range* ranges = st_stream_plan_ranges(plans[j], &nr);
        for (size_t r = 0; r < nr; ++r)
            batch.push_back(Piece{static_cast<char*>(host_blobs[j]) + ranges[r].dst, off0 + ranges[r].begin,
                                  size_t(ranges[r].end - ranges[r].begin)});
    }
    FileFd file;
    st_status status = open_checked(path, idx, file);
    if (status != ST_OK) return status;
    auto t0 = std::chrono::steady_clock::now();
    {
        Readers pool;
        if (!pool.read(file.fd, batch)) status = st_fail(ST_E_IO, "read of %s failed", path);
    }
    if (seconds_read) *seconds_read = seconds_since(t0);
    return status;
}

extern "C" st_status st_read_plan(const char* path, const st_index* idx, const st_stream_plan* plan, void* host_blob,
                                  size_t host_bytes, double* seconds_read) {
    if (!plan || !host_blob) return st_fail(ST_E_ARG, "st_read_plan: null pointer");
    return st_read_plans(path, idx, &plan, &host_blob, &host_bytes, 1, seconds_read);
}
