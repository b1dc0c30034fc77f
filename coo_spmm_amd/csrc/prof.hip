// prof.hip -- optional per-kernel-class timing with HIP events recorded on the
// launch stream around each library launch.
#include "internal.h"

#include <map>
#include <mutex>
#include <utility>

namespace snack {
namespace {

struct Rec {
    int k;
    int64_t tag;
    hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_open;          // started, not yet ended (per class, LIFO)
std::vector<Rec> g_done;          // ended, not yet read
std::vector<hipEvent_t> g_pool;   // reusable events
int64_t g_count[KC_COUNT];
double g_ms[KC_COUNT];
int64_t g_tag = 0;
std::map<std::pair<int, int64_t>, std::pair<int64_t, double>> g_tagged;

const char* const g_names[KC_COUNT] = {"spmm_forward", "spmm_dx", "sddmm_dw", "transpose", "vals_t_refresh",
                                       "sgd", "elementwise", "radix_sort", "canonicalise", "prune_regrow"};

hipEvent_t get_event()
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

void drain_locked()
{
    for (Rec& r : g_done) {
        if (r.a && r.b && hipEventSynchronize(r.b) == hipSuccess) {
            float ms = 0.0f;
            if (hipEventElapsedTime(&ms, r.a, r.b) == hipSuccess) {
                g_ms[r.k] += ms;
                g_count[r.k] += 1;
                auto key = std::make_pair(r.k, r.tag);
                if (g_tagged.count(key) || g_tagged.size() < 1024 * KC_COUNT) {
                    auto& t = g_tagged[key];
                    t.first += 1;
                    t.second += ms;
                }
            }
        }
        if (r.a) g_pool.push_back(r.a);
        if (r.b) g_pool.push_back(r.b);
    }
    g_done.clear();
}

}  // namespace

bool prof_on() { return g_on; }

void prof_begin(int kclass, hipStream_t s)
{
    std::lock_guard<std::mutex> lk(g_mu);
    Rec r{kclass, g_tag, get_event(), nullptr};
    if (r.a) hipEventRecord(r.a, s);
    g_open.push_back(r);
}

void prof_end(int kclass, hipStream_t s)
{
    std::lock_guard<std::mutex> lk(g_mu);
    for (size_t i = g_open.size(); i-- > 0;) {
        if (g_open[i].k == kclass) {
            Rec r = g_open[i];
            g_open.erase(g_open.begin() + (ptrdiff_t)i);
            r.b = get_event();
            if (r.b) hipEventRecord(r.b, s);
            g_done.push_back(r);
            // bound the number of outstanding events
            if (g_done.size() > 4096) drain_locked();
            return;
        }
    }
}

}  // namespace snack

using namespace snack;

extern "C" snack_status snack_profile_enable(int on)
{
    std::lock_guard<std::mutex> lk(g_mu);
    g_on = on != 0;
    return SNACK_OK;
}

extern "C" snack_status snack_profile_reset(void)
{
    std::lock_guard<std::mutex> lk(g_mu);
    drain_locked();
    for (int i = 0; i < KC_COUNT; ++i) {
        g_count[i] = 0;
        g_ms[i] = 0.0;
    }
    g_tagged.clear();
    return SNACK_OK;
}

extern "C" const char* snack_profile_name(int kernel_class)
{
    if (kernel_class < 0 || kernel_class >= KC_COUNT) return nullptr;
    return g_names[kernel_class];
}

extern "C" snack_status snack_profile_read(int kernel_class, int64_t* launches, double* total_ms)
{
    if (kernel_class < 0 || kernel_class >= KC_COUNT || !launches || !total_ms) return SNACK_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_mu);
    drain_locked();
    *launches = g_count[kernel_class];
    *total_ms = g_ms[kernel_class];
    return SNACK_OK;
}

extern "C" snack_status snack_profile_set_tag(int64_t tag)
{
    std::lock_guard<std::mutex> lk(g_mu);
    g_tag = tag;
    return SNACK_OK;
}

extern "C" snack_status snack_profile_read_tag(int kernel_class, int64_t tag, int64_t* launches, double* total_ms)
{
    if (kernel_class < 0 || kernel_class >= KC_COUNT || !launches || !total_ms) return SNACK_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lk(g_mu);
    drain_locked();
    auto it = g_tagged.find(std::make_pair(kernel_class, tag));
    *launches = it == g_tagged.end() ? 0 : it->second.first;
    *total_ms = it == g_tagged.end() ? 0.0 : it->second.second;
    return SNACK_OK;
}
