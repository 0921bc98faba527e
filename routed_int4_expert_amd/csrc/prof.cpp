// prof.cpp -- optional per-kernel HIP-event timing for benchmarks (moe_prof_*).
//
// While enabled, each launch site opens a ProfScope, which records a start
// event before the launch and a stop event after it on the launch's stream.
// Events are pooled and reused; nothing is allocated on the device.  The recorder
// belongs to the host thread that enabled it (thread-local): calls made on other
// threads are neither timed nor affected, and no recording changes what a call
// computes.
#include <hip/hip_runtime.h>
#include <string.h>

#include <string>
#include <vector>

#include "moe.h"
#include "moe_internal.h"

namespace moe {
namespace {

struct Rec {
    std::string name;
    hipEvent_t a, b;
};

// One recorder per host thread; never freed, so no destructor runs at thread or
// process exit (when the HIP runtime may already be gone).
struct Recorder {
    bool on = false;
    bool err = false;
    std::vector<Rec> recs;
    std::vector<hipEvent_t> pool;
};

thread_local Recorder *t_rec = nullptr;

Recorder &rec() {
    if (!t_rec) t_rec = new Recorder();
    return *t_rec;
}

hipEvent_t take_event(Recorder &r) {
    if (!r.pool.empty()) {
        hipEvent_t e = r.pool.back();
        r.pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
        r.err = true;
        return nullptr;
    }
    return e;
}

}  // namespace

ProfScope::ProfScope(const char *name, hipStream_t s) : slot(-1), st(s) {
    if (!t_rec || !t_rec->on) return;
    Recorder &r = *t_rec;
    Rec e;
    e.name = name;
    e.a = take_event(r);
    e.b = take_event(r);
    if (!e.a || !e.b || hipEventRecord(e.a, st) != hipSuccess) {
        r.err = true;
        return;
    }
    slot = (int)r.recs.size();
    r.recs.push_back(e);
}

ProfScope::~ProfScope() {
    if (slot < 0) return;
    Recorder &r = *t_rec;
    if (slot < (int)r.recs.size() && hipEventRecord(r.recs[slot].b, st) != hipSuccess) r.err = true;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_prof_begin(void) {
    Recorder &r = rec();
    for (Rec &e : r.recs) {
        r.pool.push_back(e.a);
        r.pool.push_back(e.b);
    }
    r.recs.clear();
    r.err = false;
    r.on = true;
    return MOE_OK;
}

extern "C" int moe_prof_end(moe_prof_stat *out, int32_t max_entries, int32_t *n_entries) {
    if (max_entries < 0 || (max_entries > 0 && !out) || !n_entries) return MOE_EINVAL;
    Recorder &r = rec();
    r.on = false;
    std::vector<moe_prof_stat> acc;
    bool err = r.err;
    for (Rec &e : r.recs) {
        float ms = 0.f;
        if (hipEventSynchronize(e.b) != hipSuccess || hipEventElapsedTime(&ms, e.a, e.b) != hipSuccess) {
            err = true;
            continue;
        }
        size_t i = 0;
        for (; i < acc.size(); i++)
            if (e.name == acc[i].name) break;
        if (i == acc.size()) {
            moe_prof_stat st;
            memset(&st, 0, sizeof(st));
            strncpy(st.name, e.name.c_str(), sizeof(st.name) - 1);
            acc.push_back(st);
        }
        acc[i].launches += 1;
        acc[i].ms += ms;
    }
    for (Rec &e : r.recs) {
        r.pool.push_back(e.a);
        r.pool.push_back(e.b);
    }
    r.recs.clear();
    *n_entries = (int32_t)acc.size();
    for (int i = 0; i < (int)acc.size() && i < max_entries; i++) out[i] = acc[i];
    return err ? MOE_EDEVICE : MOE_OK;
}
