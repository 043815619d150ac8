// workspace.h -- the decode workspace registry of libgqa (host-only C++, no
// HIP headers, so that the policy builds into a host unit test with g++).
//
// Split decode writes fp32 partial rows that a second kernel merges; they
// live in a block of device memory that the library keeps per (device,
// stream). The policy, with the device calls injected through WsBackend:
//  * A block is allocated on the first call that needs one and grown when a
//    later call needs more. A block that no captured graph uses is freed in
//    stream order when it is replaced.
//  * A call made while its stream is being captured into a graph never
//    allocates: it uses the stream's block if that is large enough (which
//    marks the block as referenced by a graph) and fails otherwise.
//  * A block a graph references is never freed by growth: it moves to a
//    retired list and stays valid, so replays of the graph keep working
//    after later, larger eager calls on the same stream.
//  * release_all() frees every block, live and retired, after waiting for
//    the devices that hold them; graphs captured before it must not be
//    replayed afterwards.
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

#include "gqa.h"

namespace gqa {

// Device operations the registry needs. Each returns 0 on success, else a
// nonzero code whose text error_text() gives.
struct WsBackend {
    virtual ~WsBackend() = default;
    virtual int alloc(void **ptr, int64_t bytes, void *stream) = 0;  // stream-ordered allocation
    virtual int free_async(void *ptr, void *stream) = 0;             // stream-ordered free
    virtual int free_now(int device, void *ptr) = 0;                 // after the device is idle
    virtual int sync_device(int device) = 0;
    virtual int is_capturing(void *stream, bool *capturing) = 0;
    virtual std::string error_text(int code) = 0;
};

class WorkspaceRegistry {
public:
    explicit WorkspaceRegistry(WsBackend *backend) : be_(backend) {}

    // A block of at least `bytes` for (device, stream) in *out. Not thread
    // safe: the caller holds a lock.
    gqa_status get(int device, void *stream, int64_t bytes, char **out, std::string *err);

    // Frees every block (live and retired), waiting first for each device
    // that holds one. Not thread safe: the caller holds a lock.
    gqa_status release_all(std::string *err);

    // Introspection for tests.
    int64_t live_bytes(int device, void *stream) const;
    bool live_captured(int device, void *stream) const;
    size_t retired_count() const { return retired_.size(); }
    size_t live_count() const { return live_.size(); }

private:
    struct Key {
        int device;
        void *stream;
        bool operator==(const Key &o) const { return device == o.device && stream == o.stream; }
    };
    struct KeyHash {
        size_t operator()(const Key &k) const
        {
            return std::hash<void *>()(k.stream) * 31u + static_cast<size_t>(k.device);
        }
    };
    struct Block {
        char *ptr = nullptr;
        int64_t bytes = 0;
        bool captured = false;  // referenced by a captured graph
    };
    struct Retired {
        int device;
        char *ptr;
    };

    WsBackend *be_;
    std::unordered_map<Key, Block, KeyHash> live_;
    std::vector<Retired> retired_;
};

}  // namespace gqa
