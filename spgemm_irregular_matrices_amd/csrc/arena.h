// Plan-owned device workspace: named buffers that only grow.
#pragma once

#include <hip/hip_runtime.h>

#include <string>
#include <type_traits>
#include <unordered_map>

#include "common.h"

namespace sg {

class Arena {
  public:
    Arena() = default;
    Arena(const Arena&) = delete;
    Arena& operator=(const Arena&) = delete;
    ~Arena() { release(); }

    // Largest total the arena may hold (0 = no limit). A request that would
    // pass it fails as if the device had no more memory.
    void set_limit(size_t bytes) { limit_ = bytes; }

    // Debug aid: floating-point buffers are filled with NaN (all bits set)
    // when they are allocated, so that a read of workspace nothing wrote
    // shows up in the results. Index buffers are left alone: a poisoned
    // index would send a kernel outside its arrays. Not with a region (that
    // mode promises no calls beyond the caller's kernels).
    void set_poison(bool on) { poison_ = on; }

    // Carve every buffer out of the device range [base, base + bytes)
    // instead of allocating: while a region is set the arena calls neither
    // hipMalloc nor hipFree. Buffers are laid out one after the other in
    // the order they are first asked for; a buffer asked for again with more
    // room moves to the end (its contents are not kept, as when a heap
    // buffer grows), and release() forgets them all.
    void use_region(void* base, size_t bytes) {
        release();
        region_ = static_cast<char*>(base);
        region_cap_ = bytes;
    }

    // Device buffer `name` with room for at least `bytes`. Growing frees the
    // old buffer (hipFree waits for the device, so no kernel still uses it).
    void* get(const std::string& name, size_t bytes, bool* fresh = nullptr) {
        if (fresh) *fresh = false;
        Buf& b = bufs_[name];
        if (bytes == 0) bytes = 1;
        if (region_ && b.cap < bytes) {
            const size_t off = (total_ + 255) & ~size_t(255);
            const size_t cap = (bytes + 255) & ~size_t(255);
            if (off > region_cap_ || cap > region_cap_ - off)
                throw ScratchError("workspace '" + name + "' (" + std::to_string(bytes) +
                                   " bytes) does not fit the fixed scratch buffer");
            b.p = region_ + off;
            b.cap = cap;
            total_ = off + cap;
        }
        if (b.cap < bytes) {
            if (b.p) {
                (void)hipFree(b.p);
                total_ -= b.cap;
                b.p = nullptr;
                b.cap = 0;
            }
            size_t extra = bytes / 8;
            if (extra > (size_t(256) << 20)) extra = size_t(256) << 20;
            size_t cap = (bytes + extra + (size_t(2) << 20) - 1) & ~((size_t(2) << 20) - 1);
            if (limit_ && total_ + cap > limit_) cap = (bytes + 255) & ~size_t(255);
            if (limit_ && total_ + cap > limit_)
                throw OomError("device workspace '" + name + "' (" + std::to_string(bytes) +
                               " bytes) passes the plan's workspace limit");
            void* p = nullptr;
            if (hipMalloc(&p, cap) != hipSuccess) {
                (void)hipGetLastError();
                // retry without headroom before giving up
                cap = (bytes + 255) & ~size_t(255);
                if (hipMalloc(&p, cap) != hipSuccess) {
                    (void)hipGetLastError();
                    throw OomError("device workspace '" + name + "' (" + std::to_string(bytes) +
                                   " bytes)");
                }
            }
            b.p = p;
            b.cap = cap;
            total_ += cap;
            if (fresh) *fresh = true;
        }
        return b.p;
    }

    template <class T>
    T* get(const std::string& name, size_t count) {
        bool fresh = false;
        T* p = static_cast<T*>(get(name, count * sizeof(T), &fresh));
        if constexpr (std::is_floating_point<T>::value) {
            if (fresh && poison_ && !region_) {
                if (hipMemset(p, 0xff, bufs_[name].cap) != hipSuccess ||
                    hipDeviceSynchronize() != hipSuccess)
                    throw HipError(hipGetLastError(), "poisoning a workspace buffer");
            }
        }
        return p;
    }

    size_t total_bytes() const { return total_; }

    void release() {
        if (!region_)
            for (auto& kv : bufs_)
                if (kv.second.p) (void)hipFree(kv.second.p);
        bufs_.clear();
        total_ = 0;
    }

  private:
    struct Buf {
        void* p = nullptr;
        size_t cap = 0;
    };
    std::unordered_map<std::string, Buf> bufs_;
    size_t total_ = 0;  // bytes held (with a region: the end of its last buffer)
    size_t limit_ = 0;
    bool poison_ = false;
    char* region_ = nullptr;
    size_t region_cap_ = 0;
};

}  // namespace sg
