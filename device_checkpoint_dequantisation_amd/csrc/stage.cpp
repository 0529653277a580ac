// Staging: the file's data section -> pinned host ring -> one device blob.
//
// The pages ("Disk tier safetensors streaming design audit", "Strategy summary / Range reads
// and tiering") read only a tensor's byte range into (optionally pinned) host memory, copy it
// to the GPU and release the host buffer.  Here the whole data section is one range: it is read
// in chunks by a few threads into a ring carved from the caller's pinned buffer, and each chunk
// is copied with hipMemcpyAsync on a side stream while the next chunk is being read.  An event
// per ring slot keeps a slot from being overwritten before its copy has finished.
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <thread>
#include <vector>

#include "st_internal.h"

namespace {

constexpr size_t kMinPinned = size_t(2) << 20;
constexpr int kSlots = 4;
constexpr int kReaders = 8;

// Reads [off, off + len) of fd into dst with `kReaders` threads; false on a short read.
bool read_range(int fd, char* dst, uint64_t off, size_t len) {
    std::atomic<bool> ok{true};
    auto piece = [&](size_t b, size_t e) {
        while (b < e) {
            ssize_t r = pread(fd, dst + b, e - b, off_t(off + b));
            if (r <= 0) { ok = false; return; }
            b += size_t(r);
        }
    };
    const size_t min_piece = size_t(4) << 20;
    int nt = int(std::min<size_t>(kReaders, std::max<size_t>(1, len / min_piece)));
    if (nt == 1) {
        piece(0, len);
        return ok;
    }
    std::vector<std::thread> th;
    size_t step = (len + size_t(nt) - 1) / size_t(nt);
    step = (step + 4095) & ~size_t(4095);
    for (size_t b = 0; b < len; b += step) th.emplace_back(piece, b, std::min(len, b + step));
    for (auto& t : th) t.join();
    return ok;
}

}  // namespace

extern "C" st_status st_stage_file(const char* path, const st_index* idx, void* blob_dev, void* pinned,
                                   size_t pinned_bytes, void* side_stream, void* done_event, double* seconds_read) {
    if (!path || !idx || !blob_dev || !pinned) return st_fail(ST_E_ARG, "st_stage_file: null pointer");
    if (pinned_bytes < kMinPinned)
        return st_fail(ST_E_ARG, "st_stage_file: pinned buffer of %zu bytes, at least %zu needed", pinned_bytes, kMinPinned);
    if (reinterpret_cast<uintptr_t>(blob_dev) % ST_BLOB_ALIGN)
        return st_fail(ST_E_ARG, "st_stage_file: blob is not %d-byte aligned", ST_BLOB_ALIGN);
    const uint64_t off0 = st_index_data_offset(idx), size = st_index_data_size(idx);
    int fd = open(path, O_RDONLY | O_CLOEXEC);
    if (fd < 0) return st_fail(ST_E_IO, "cannot open %s", path);
    struct stat sb;
    if (fstat(fd, &sb) != 0 || uint64_t(sb.st_size) != off0 + size) {
        close(fd);
        return st_fail(ST_E_IO, "%s is %lld bytes, the index expects %llu", path, (long long)sb.st_size,
                       (unsigned long long)(off0 + size));
    }
    hipStream_t stream = static_cast<hipStream_t>(side_stream);
    size_t chunk = (pinned_bytes / kSlots) & ~size_t(4095);
    hipEvent_t ev[kSlots];
    for (int s = 0; s < kSlots; ++s)
        if (hipEventCreateWithFlags(&ev[s], hipEventDisableTiming) != hipSuccess) {
            for (int k = 0; k < s; ++k) (void)hipEventDestroy(ev[k]);
            close(fd);
            return st_fail(ST_E_HIP, "st_stage_file: hipEventCreate failed");
        }
    st_status status = ST_OK;
    double t_read = 0;
    uint64_t done = 0;
    for (uint64_t i = 0; done < size; ++i) {
        int s = int(i % kSlots);
        char* slot = static_cast<char*>(pinned) + size_t(s) * chunk;
        size_t len = size_t(std::min<uint64_t>(chunk, size - done));
        if (i >= kSlots && hipEventSynchronize(ev[s]) != hipSuccess) {
            status = st_fail(ST_E_HIP, "st_stage_file: waiting for a staging copy failed");
            break;
        }
        auto t0 = std::chrono::steady_clock::now();
        bool ok = read_range(fd, slot, off0 + done, len);
        t_read += std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
        if (!ok) {
            status = st_fail(ST_E_IO, "read of %s failed at byte %llu", path, (unsigned long long)(off0 + done));
            break;
        }
        if (hipMemcpyAsync(static_cast<char*>(blob_dev) + done, slot, len, hipMemcpyHostToDevice, stream) != hipSuccess ||
            hipEventRecord(ev[s], stream) != hipSuccess) {
            status = st_fail(ST_E_HIP, "st_stage_file: hipMemcpyAsync of %zu bytes failed", len);
            break;
        }
        done += len;
    }
    close(fd);
    if (status == ST_OK && done_event && hipEventRecord(static_cast<hipEvent_t>(done_event), stream) != hipSuccess)
        status = st_fail(ST_E_HIP, "st_stage_file: hipEventRecord failed");
    if (status != ST_OK) (void)hipStreamSynchronize(stream);  // nothing may still read the ring
    for (int s = 0; s < kSlots; ++s) (void)hipEventDestroy(ev[s]);
    if (seconds_read) *seconds_read = t_read;
    return status;
}
