// prof.cpp -- optional per-kernel HIP-event timing for benchmarks (moe_prof_*).
//
// While enabled, each launch site opens a ProfScope, which records a start
// event before the launch and a stop event after it on the launch's stream.
// Events are pooled and reused; nothing is allocated on the device.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>
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

std::mutex g_mu;
bool g_on = false;
bool g_err = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
        g_err = true;
        return nullptr;
    }
    return e;
}

}  // namespace

ProfScope::ProfScope(const char *name, hipStream_t s) : slot(-1), st(s) {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on) return;
    Rec r;
    r.name = name;
    r.a = take_event();
    r.b = take_event();
    if (!r.a || !r.b || hipEventRecord(r.a, st) != hipSuccess) {
        g_err = true;
        return;
    }
    slot = (int)g_recs.size();
    g_recs.push_back(r);
}

ProfScope::~ProfScope() {
    if (slot < 0) return;
    std::lock_guard<std::mutex> lk(g_mu);
    if (slot < (int)g_recs.size() && hipEventRecord(g_recs[slot].b, st) != hipSuccess) g_err = true;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_prof_begin(void) {
    std::lock_guard<std::mutex> lk(g_mu);
    for (Rec &r : g_recs) {
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
    g_err = false;
    g_on = true;
    return MOE_OK;
}

extern "C" int moe_prof_end(moe_prof_stat *out, int32_t max_entries, int32_t *n_entries) {
    if (max_entries < 0 || (max_entries > 0 && !out) || !n_entries) return MOE_EINVAL;
    std::lock_guard<std::mutex> lk(g_mu);
    g_on = false;
    std::vector<moe_prof_stat> acc;
    bool err = g_err;
    for (Rec &r : g_recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
            err = true;
            continue;
        }
        size_t i = 0;
        for (; i < acc.size(); i++)
            if (r.name == acc[i].name) break;
        if (i == acc.size()) {
            moe_prof_stat s;
            memset(&s, 0, sizeof(s));
            strncpy(s.name, r.name.c_str(), sizeof(s.name) - 1);
            acc.push_back(s);
        }
        acc[i].launches += 1;
        acc[i].ms += ms;
    }
    for (Rec &r : g_recs) {
        g_pool.push_back(r.a);
        g_pool.push_back(r.b);
    }
    g_recs.clear();
    *n_entries = (int32_t)acc.size();
    for (int i = 0; i < (int)acc.size() && i < max_entries; i++) out[i] = acc[i];
    return err ? MOE_EDEVICE : MOE_OK;
}
