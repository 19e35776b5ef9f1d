// profile.cpp -- optional per-kernel timing with HIP events (hstu_profile_*).
#include "../../include/hstu.h"
#include "profile.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

namespace {

struct Pending {
    const char *name;
    hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event()
{
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

} // namespace

ProfScope::ProfScope(const char *name, hipStream_t st) : name_(name), st_(st)
{
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_on) return;
    a_ = take_event();
    if (a_) hipEventRecord((hipEvent_t)a_, st_);
}

ProfScope::~ProfScope()
{
    if (!a_) return;
    std::lock_guard<std::mutex> lk(g_mu);
    hipEvent_t b = take_event();
    if (!b) return;
    hipEventRecord(b, st_);
    g_pending.push_back(Pending{name_, (hipEvent_t)a_, b});
}

extern "C" void hstu_profile_enable(int32_t on)
{
    std::lock_guard<std::mutex> lk(g_mu);
    g_on = on != 0;
}

extern "C" int32_t hstu_profile_collect(hstu_kernel_time *out, int32_t cap)
{
    std::lock_guard<std::mutex> lk(g_mu);
    std::map<std::string, std::pair<int, double>> agg;
    std::vector<std::string> order;
    for (const Pending &p : g_pending) {
        hipEventSynchronize(p.b);
        float ms = 0.f;
        hipEventElapsedTime(&ms, p.a, p.b);
        auto it = agg.find(p.name);
        if (it == agg.end()) {
            order.push_back(p.name);
            agg[p.name] = {1, (double)ms};
        } else {
            it->second.first++;
            it->second.second += ms;
        }
        g_pool.push_back(p.a);
        g_pool.push_back(p.b);
    }
    g_pending.clear();
    int n = 0;
    for (const std::string &name : order) {
        if (n >= cap) break;
        std::memset(out[n].name, 0, sizeof out[n].name);
        std::strncpy(out[n].name, name.c_str(), sizeof out[n].name - 1);
        out[n].launches = agg[name].first;
        out[n].total_ms = agg[name].second;
        n++;
    }
    return n;
}
