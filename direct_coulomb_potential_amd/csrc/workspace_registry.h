// Host-side record of the workspaces the library has filled (plain C++, no
// HIP: the host tests build it on its own).
//
// cpmap_bin_atoms and cpmap_bin_slots fill a caller-owned workspace that a
// later cutoff call reads.  The registry remembers, per workspace, the range
// the library wrote, what it was filled for (atom count, lattice, bin
// geometry, slot capacity) and a number that the same call also writes into
// the workspace's device header.  A cutoff call accepts a workspace only if a
// record with its exact base address, kind, size and key exists; every call
// that writes device memory first drops each record whose range overlaps a
// range it writes, so a workspace rebinned through another base address, or
// used as scratch or output by any entry point, is refused afterwards.
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstring>
#include <iterator>
#include <map>
#include <mutex>

namespace cpmap {

// What a workspace was filled for.  Compared byte for byte (padding zeroed).
struct WorkspaceKey {
    int64_t n_atoms;
    int32_t n[3];
    float h, o[3], bs, rc;
    int32_t cap;  // slots per bin; 0 for a binned (CSR) workspace

    static WorkspaceKey make(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz, float h,
                             float ox, float oy, float oz, float bs, float rc, int32_t cap)
    {
        WorkspaceKey k;
        std::memset(&k, 0, sizeof k);
        k.n_atoms = n_atoms;
        k.n[0] = nx;
        k.n[1] = ny;
        k.n[2] = nz;
        k.h = h;
        k.o[0] = ox;
        k.o[1] = oy;
        k.o[2] = oz;
        k.bs = bs;
        k.rc = rc;
        k.cap = cap;
        return k;
    }
    bool operator==(const WorkspaceKey &k) const { return std::memcmp(this, &k, sizeof k) == 0; }
};

enum WorkspaceKind { kBinnedWorkspace = 1, kSlotWorkspace = 2 };

class WorkspaceRegistry {
  public:
    // Drops every record whose range overlaps [p, p + bytes).
    void forget(const void *p, size_t bytes)
    {
        if (p == nullptr || bytes == 0)
            return;
        std::lock_guard<std::mutex> lock(mu_);
        forget_locked(reinterpret_cast<uintptr_t>(p), bytes);
    }

    // Records that [p, p + bytes) now holds a workspace of this kind filled
    // for key (dropping the records it overlaps); returns the fill's number,
    // never 0.
    uint64_t record(const void *p, size_t bytes, WorkspaceKind kind, const WorkspaceKey &key)
    {
        const uintptr_t a = reinterpret_cast<uintptr_t>(p);
        std::lock_guard<std::mutex> lock(mu_);
        forget_locked(a, bytes);
        const uint64_t nonce = next_++;
        entries_[a] = Entry{bytes, kind, key, nonce};
        return nonce;
    }

    // The number of the fill recorded at exactly p with this kind, size and
    // key, or 0 when there is none.
    uint64_t find(const void *p, size_t bytes, WorkspaceKind kind, const WorkspaceKey &key) const
    {
        std::lock_guard<std::mutex> lock(mu_);
        auto it = entries_.find(reinterpret_cast<uintptr_t>(p));
        if (it == entries_.end() || it->second.bytes != bytes || it->second.kind != kind ||
            !(it->second.key == key))
            return 0;
        return it->second.nonce;
    }

    size_t size() const
    {
        std::lock_guard<std::mutex> lock(mu_);
        return entries_.size();
    }

  private:
    struct Entry {
        size_t bytes;
        WorkspaceKind kind;
        WorkspaceKey key;
        uint64_t nonce;
    };

    // Records never overlap one another, so only the last record starting at
    // or before a can reach into [a, a + bytes); the others overlapping it
    // start inside it.
    void forget_locked(uintptr_t a, size_t bytes)
    {
        const uintptr_t end = a + bytes < a ? UINTPTR_MAX : a + bytes;
        auto it = entries_.upper_bound(a);
        if (it != entries_.begin()) {
            auto prev = std::prev(it);
            if (prev->first + prev->second.bytes > a)
                it = prev;
        }
        while (it != entries_.end() && it->first < end)
            it = entries_.erase(it);
    }

    mutable std::mutex mu_;
    std::map<uintptr_t, Entry> entries_;
    uint64_t next_ = 1;
};

}  // namespace cpmap
