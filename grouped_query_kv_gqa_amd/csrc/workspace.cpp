// workspace.cpp -- decode workspace registry policy (host-only; see workspace.h).
#include "workspace.h"

#include <set>

namespace gqa {

namespace {

gqa_status fail(std::string *err, gqa_status s, const std::string &msg)
{
    if (err)
        *err = msg;
    return s;
}

}  // namespace

gqa_status WorkspaceRegistry::get(int device, void *stream, int64_t bytes, char **out, std::string *err)
{
    *out = nullptr;
    if (bytes <= 0)
        return GQA_OK;
    bool capturing = false;
    int e = be_->is_capturing(stream, &capturing);
    if (e != 0)
        return fail(err, GQA_ERR_HIP, "stream capture query: " + be_->error_text(e));
    const Key key{device, stream};
    auto it = live_.find(key);
    if (capturing) {
        if (it == live_.end() || it->second.bytes < bytes)
            return fail(err, GQA_ERR_INVALID_ARG,
                        "the decode workspace of this stream is missing or too small and cannot be allocated "
                        "while the stream is being captured; make one call of the same or a larger shape on "
                        "the stream before capturing");
        it->second.captured = true;
        *out = it->second.ptr;
        return GQA_OK;
    }
    if (it != live_.end() && it->second.bytes >= bytes) {
        *out = it->second.ptr;
        return GQA_OK;
    }
    // Allocate the new block before giving up the old one, so that a failed
    // allocation leaves the registry as it was.
    const int64_t grown = bytes + bytes / 4;  // headroom for growth
    void *p = nullptr;
    e = be_->alloc(&p, grown, stream);
    if (e != 0)
        return fail(err, GQA_ERR_HIP, "workspace allocation: " + be_->error_text(e));
    if (it != live_.end()) {
        Block &old = it->second;
        if (old.captured) {
            retired_.push_back({device, old.ptr});
        } else {
            e = be_->free_async(old.ptr, stream);
            if (e != 0) {
                // keep the old block alive rather than lose track of it
                retired_.push_back({device, old.ptr});
            }
        }
        old = Block{};
    }
    Block &blk = live_[key];
    blk.ptr = static_cast<char *>(p);
    blk.bytes = grown;
    blk.captured = false;
    *out = blk.ptr;
    return GQA_OK;
}

gqa_status WorkspaceRegistry::release_all(std::string *err)
{
    std::set<int> devices;
    for (const auto &kv : live_)
        devices.insert(kv.first.device);
    for (const auto &r : retired_)
        devices.insert(r.device);
    for (int d : devices) {
        int e = be_->sync_device(d);
        if (e != 0)
            return fail(err, GQA_ERR_HIP, "device synchronisation: " + be_->error_text(e));
    }
    gqa_status st = GQA_OK;
    for (const auto &kv : live_) {
        int e = be_->free_now(kv.first.device, kv.second.ptr);
        if (e != 0 && st == GQA_OK)
            st = fail(err, GQA_ERR_HIP, "workspace free: " + be_->error_text(e));
    }
    for (const auto &r : retired_) {
        int e = be_->free_now(r.device, r.ptr);
        if (e != 0 && st == GQA_OK)
            st = fail(err, GQA_ERR_HIP, "workspace free: " + be_->error_text(e));
    }
    live_.clear();
    retired_.clear();
    return st;
}

int64_t WorkspaceRegistry::live_bytes(int device, void *stream) const
{
    auto it = live_.find(Key{device, stream});
    return it == live_.end() ? 0 : it->second.bytes;
}

bool WorkspaceRegistry::live_captured(int device, void *stream) const
{
    auto it = live_.find(Key{device, stream});
    return it != live_.end() && it->second.captured;
}

}  // namespace gqa
