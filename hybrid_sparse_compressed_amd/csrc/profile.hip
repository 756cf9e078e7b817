// profile.hip -- optional per-kernel timing with HIP events.
//
// When a kernel family is armed (hsa_profile_enable), every launch of that
// family is bracketed by two hipEventRecord calls on the launch stream; the
// pairs come from a fixed pool created on the first arm.  hsa_profile_read
// waits for the recorded pairs, sums their elapsed times per family and
// returns the pairs to the pool.  Nothing is recorded while no family is
// armed, so the hot path pays one relaxed atomic load per launch.
#include "../../include/hsa_attn.h"
#include "hsa_internal.hpp"

#include <atomic>
#include <mutex>
#include <vector>

namespace hsa {

namespace {

constexpr int kFamilies = 8;
constexpr int kPool = 8192;

struct Pending {
    int family;
    int slot;
};

struct ProfState {
    std::mutex mu;
    std::vector<hipEvent_t> ev;  // 2 per slot
    std::vector<int> free_slots;
    std::vector<Pending> pending;
    double total_ms[kFamilies] = {};
    long long launches[kFamilies] = {};
    int device = -1;
};

std::atomic<unsigned> g_mask{0};
ProfState& state() {
    static ProfState s;
    return s;
}

int family_index(unsigned fam) {
    for (int i = 0; i < kFamilies; ++i)
        if (fam == (1u << i)) return i;
    return -1;
}

}  // namespace

ProfScope::ProfScope(unsigned family, hipStream_t st) : family_(family), st_(st), slot_(-1) {
    if ((g_mask.load(std::memory_order_relaxed) & family) == 0) return;
    ProfState& s = state();
    std::lock_guard<std::mutex> lk(s.mu);
    if (s.free_slots.empty()) return;  // pool exhausted: this launch is not timed
    slot_ = s.free_slots.back();
    s.free_slots.pop_back();
    if (hipEventRecord(s.ev[2 * slot_], st_) != hipSuccess) {
        s.free_slots.push_back(slot_);
        slot_ = -1;
    }
}

ProfScope::~ProfScope() {
    if (slot_ < 0) return;
    ProfState& s = state();
    std::lock_guard<std::mutex> lk(s.mu);
    if (hipEventRecord(s.ev[2 * slot_ + 1], st_) != hipSuccess) {
        s.free_slots.push_back(slot_);
        return;
    }
    s.pending.push_back(Pending{family_index(family_), slot_});
}

}  // namespace hsa

extern "C" {

int hsa_profile_enable(unsigned family_mask) {
    hsa::ProfState& s = hsa::state();
    std::lock_guard<std::mutex> lk(s.mu);
    if (family_mask != 0 && s.ev.empty()) {
        s.ev.resize(2 * hsa::kPool);
        for (auto& e : s.ev)
            // timing only: no system-scope fence (cache write-back and
            // invalidate) when the event is recorded, so the pair brackets
            // the kernel and not the fence
            if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess)
                return HSA_ERR_HIP;
        for (int i = hsa::kPool - 1; i >= 0; --i) s.free_slots.push_back(i);
    }
    hsa::g_mask.store(family_mask, std::memory_order_relaxed);
    return HSA_OK;
}

int hsa_profile_read(unsigned family, double* total_ms, long long* launches, int reset) {
    const int fi = hsa::family_index(family);
    if (fi < 0 || !total_ms || !launches) return HSA_ERR_INVALID_ARG;
    hsa::ProfState& s = hsa::state();
    std::lock_guard<std::mutex> lk(s.mu);
    for (const hsa::Pending& p : s.pending) {
        hipEvent_t a = s.ev[2 * p.slot], b = s.ev[2 * p.slot + 1];
        if (hipEventSynchronize(b) != hipSuccess) return HSA_ERR_HIP;
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return HSA_ERR_HIP;
        if (p.family >= 0) {
            s.total_ms[p.family] += ms;
            s.launches[p.family] += 1;
        }
        s.free_slots.push_back(p.slot);
    }
    s.pending.clear();
    *total_ms = s.total_ms[fi];
    *launches = s.launches[fi];
    if (reset) {
        for (int i = 0; i < hsa::kFamilies; ++i) {
            s.total_ms[i] = 0.0;
            s.launches[i] = 0;
        }
    }
    return HSA_OK;
}

}  // extern "C"
