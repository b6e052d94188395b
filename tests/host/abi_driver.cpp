// Host-only driver of the C ABI for the sanitizer builds (see
// stub_launch.cpp): every validation path with fake, never dereferenced
// device addresses, valid calls that reach the (stub) launchers in stage
// order, and the queries called from many threads at once.  Prints "ok" and
// exits 0 when every check holds.
#include <atomic>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "../../include/ssd.h"

extern std::atomic<long> g_launches[5];
extern std::atomic<long> g_event_records;

static int g_fail = 0;
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++g_fail;                                                     \
        }                                                                 \
    } while (0)

static ssd_shape shape(int64_t b, int64_t L, int64_t nh, int64_t p, int64_t n, int64_t g, int dtype,
                       uint32_t flags = 0, int ydtype = SSD_DTYPE_F32) {
    ssd_shape s;
    std::memset(&s, 0, sizeof(s));
    s.batch = b; s.seqlen = L; s.nheads = nh; s.headdim = p; s.dstate = n; s.ngroups = g;
    s.dtype = dtype; s.flags = flags; s.y_dtype = ydtype; s.reserved = 0;
    return s;
}

// Disjoint, 256-byte aligned fake device addresses, far apart.
struct Fake {
    uintptr_t base = (uintptr_t)1 << 44;
    void *operator()(uintptr_t off = 0) {
        base += (uintptr_t)64 << 30;
        return (void *)(base + off);
    }
};

struct Args {
    void *x, *dt, *A, *B, *C, *D, *init, *y, *fin, *ws;
    size_t ws_bytes;
};

static Args args_for(const ssd_shape &s, int64_t T, Fake &f) {
    Args a{f(), f(), f(), f(), f(), f(), nullptr, f(), f(), f(), 0};
    a.ws_bytes = ssd_chunk_scan_fwd_workspace_size(&s, T);
    return a;
}

static ssd_status fwd(const ssd_shape &s, int64_t T, const Args &a, const ssd_plan *plan = nullptr,
                      void *const *events = nullptr) {
    return ssd_chunk_scan_fwd_ex(&s, a.x, a.dt, (const float *)a.A, a.B, a.C, (const float *)a.D, T,
                                 (const float *)a.init, a.y, (float *)a.fin, a.ws, a.ws_bytes, nullptr,
                                 plan, events);
}

static long launches() {
    return g_launches[0] + g_launches[1] + g_launches[2] + g_launches[3] + g_launches[4];
}

static void validation_paths() {
    Fake f;
    const ssd_shape good = shape(2, 1000, 8, 64, 128, 2, SSD_DTYPE_BF16);
    const long before = launches();
    // required pointers
    for (int k = 0; k < 6; ++k) {
        Args a = args_for(good, 256, f);
        void **slots[] = {&a.x, &a.dt, &a.A, &a.B, &a.C, &a.y};
        *slots[k] = nullptr;
        CHECK(fwd(good, 256, a) == SSD_ERROR_INVALID_VALUE);
    }
    // shapes
    {
        ssd_shape s = shape(2, 1000, 6, 64, 128, 4, SSD_DTYPE_BF16);
        Args a = args_for(good, 256, f);
        CHECK(fwd(s, 256, a) == SSD_ERROR_INVALID_VALUE);
        s = shape(2, 1000, 8, 48, 128, 2, SSD_DTYPE_BF16);
        CHECK(fwd(s, 256, a) == SSD_ERROR_UNSUPPORTED);
        CHECK(fwd(good, 100, a) == SSD_ERROR_UNSUPPORTED);
        CHECK(ssd_chunk_scan_fwd_ex(nullptr, a.x, a.dt, nullptr, a.B, a.C, nullptr, 256, nullptr, a.y,
                                    nullptr, a.ws, a.ws_bytes, nullptr, nullptr, nullptr) ==
              SSD_ERROR_INVALID_VALUE);
        s = good;
        s.reserved = 3;
        CHECK(fwd(s, 256, a) == SSD_ERROR_INVALID_VALUE);
        s = good;
        s.flags = 8;
        CHECK(fwd(s, 256, a) == SSD_ERROR_INVALID_VALUE);
        s = shape(1, INT64_C(1) << 40, 1 << 20, 128, 256, 1, SSD_DTYPE_F32);  // element counts overflow
        CHECK(fwd(s, 256, a) == SSD_ERROR_UNSUPPORTED);
        CHECK(ssd_chunk_scan_fwd_workspace_size(&s, 256) == 0);
    }
    // workspace
    {
        Args a = args_for(good, 256, f);
        a.ws_bytes -= 1;
        CHECK(fwd(good, 256, a) == SSD_ERROR_WORKSPACE);
        a = args_for(good, 256, f);
        a.ws = nullptr;
        CHECK(fwd(good, 256, a) == SSD_ERROR_WORKSPACE);
    }
    // alignment
    {
        Args a = args_for(good, 256, f);
        a.x = (char *)a.x + 8;
        CHECK(fwd(good, 256, a) == SSD_ERROR_MISALIGNED);
        a = args_for(good, 256, f);
        a.ws = (char *)a.ws + 128;
        CHECK(fwd(good, 256, a) == SSD_ERROR_MISALIGNED);
        a = args_for(good, 256, f);
        a.fin = (char *)a.fin + 4;
        CHECK(fwd(good, 256, a) == SSD_ERROR_MISALIGNED);
    }
    // aliasing
    {
        Args a = args_for(good, 256, f);
        a.y = a.x;
        CHECK(fwd(good, 256, a) == SSD_ERROR_INVALID_VALUE);
        a = args_for(good, 256, f);
        a.B = a.ws;
        CHECK(fwd(good, 256, a) == SSD_ERROR_INVALID_VALUE);
        a = args_for(good, 256, f);
        a.init = f();
        a.fin = (char *)a.init + 256;
        CHECK(fwd(good, 256, a) == SSD_ERROR_INVALID_VALUE);
    }
    // plans
    {
        Args a = args_for(good, 256, f);
        ssd_plan p;
        CHECK(ssd_chunk_scan_fwd_default_plan(&good, 256, &p) == SSD_OK);
        ssd_plan bad = p;
        bad.chunk_out_heads = 0;
        CHECK(fwd(good, 256, a, &bad) == SSD_ERROR_INVALID_VALUE);
        bad = p;
        bad.chunk_state_heads = 5;  // 4 heads per group
        CHECK(fwd(good, 256, a, &bad) == SSD_ERROR_INVALID_VALUE);
        bad = p;
        bad.reserved[3] = 1;
        CHECK(fwd(good, 256, a, &bad) == SSD_ERROR_INVALID_VALUE);
        bad = p;
        bad.state_path = 7;
        CHECK(fwd(good, 256, a, &bad) == SSD_ERROR_INVALID_VALUE);
    }
    // events: any NULL event handle is rejected
    {
        Args a = args_for(good, 256, f);
        void *ev[8];
        for (int i = 0; i < 8; ++i) ev[i] = f();
        ev[5] = nullptr;
        CHECK(fwd(good, 256, a, nullptr, ev) == SSD_ERROR_INVALID_VALUE);
        CHECK(ssd_chunk_scan_fwd_profiled(&good, a.x, a.dt, (const float *)a.A, a.B, a.C, nullptr, 256,
                                          nullptr, a.y, nullptr, a.ws, a.ws_bytes, nullptr,
                                          nullptr) == SSD_ERROR_INVALID_VALUE);
    }
    // no-allocation entry point: shape checks and the scratch limit come first
    {
        const ssd_shape big = shape(8, 4096, 80, 64, 128, 1, SSD_DTYPE_BF16);
        Args a = args_for(big, 256, f);
        CHECK(ssd_chunk_scan_fwd_workspace_size(&big, 256) > (size_t)SSD_NOALLOC_SCRATCH_BYTES);
    }
    // decode step: seqlen must be 1, pointers present, aligned, not aliased
    {
        const ssd_shape d1 = shape(4, 1, 8, 64, 128, 2, SSD_DTYPE_BF16);
        void *x = f(), *dt = f(), *A = f(), *B = f(), *C = f(), *D = f(), *st = f(), *y = f();
        auto dec = [&](const ssd_shape &s) {
            return ssd_decode_step(&s, x, dt, (const float *)A, B, C, (const float *)D, (float *)st, y,
                                   nullptr, nullptr);
        };
        CHECK(dec(shape(4, 2, 8, 64, 128, 2, SSD_DTYPE_BF16)) == SSD_ERROR_INVALID_VALUE);
        CHECK(dec(shape(4, 1, 8, 48, 128, 2, SSD_DTYPE_BF16)) == SSD_ERROR_UNSUPPORTED);
        CHECK(dec(shape(4, 1, 8, 64, 128, 2, SSD_DTYPE_BF16, 1)) == SSD_ERROR_INVALID_VALUE);
        void *keep = st;
        st = nullptr;
        CHECK(dec(d1) == SSD_ERROR_INVALID_VALUE);
        st = (char *)keep + 8;
        CHECK(dec(d1) == SSD_ERROR_MISALIGNED);
        st = keep;
        void *keepy = y;
        y = (char *)st + 64;  // y inside the state
        CHECK(dec(d1) == SSD_ERROR_INVALID_VALUE);
        y = keepy;
        void *ev[2] = {f(), nullptr};
        CHECK(ssd_decode_step(&d1, x, dt, (const float *)A, B, C, nullptr, (float *)st, y, nullptr, ev) ==
              SSD_ERROR_INVALID_VALUE);
    }
    CHECK(launches() == before);  // nothing was enqueued by any rejected call
}

static void valid_calls() {
    Fake f;
    // every stage in order for a problem with tokens
    for (int dtype : {SSD_DTYPE_F32, SSD_DTYPE_BF16}) {
        const ssd_shape s = shape(2, 1000, 8, 64, 128, 2, dtype);
        Args a = args_for(s, 128, f);
        long c[4];
        for (int i = 0; i < 4; ++i) c[i] = g_launches[i];
        CHECK(fwd(s, 128, a) == SSD_OK);
        for (int i = 0; i < 4; ++i) CHECK(g_launches[i] == c[i] + 1);
        uint32_t m = 0;
        CHECK(ssd_chunk_scan_fwd_stage_launches(&s, 128, nullptr, &m) == SSD_OK && m == 15u);
        // profiled: stages with kernels record their events inside the
        // launch, so no separate record happens here
        void *ev[8];
        for (int i = 0; i < 8; ++i) ev[i] = f();
        const long r = g_event_records;
        CHECK(fwd(s, 128, a, nullptr, ev) == SSD_OK);
        CHECK(g_event_records == r);
    }
    // no tokens: the state pass alone, the other stages' events back to back
    {
        const ssd_shape s = shape(2, 0, 8, 64, 128, 2, SSD_DTYPE_BF16);
        Args a = args_for(s, 64, f);
        long c[4];
        for (int i = 0; i < 4; ++i) c[i] = g_launches[i];
        void *ev[8];
        for (int i = 0; i < 8; ++i) ev[i] = f();
        const long r = g_event_records;
        CHECK(fwd(s, 64, a, nullptr, ev) == SSD_OK);
        CHECK(g_launches[0] == c[0] && g_launches[1] == c[1] && g_launches[2] == c[2] + 1 &&
              g_launches[3] == c[3]);
        CHECK(g_event_records == r + 6);
    }
    // empty batch: nothing at all, no pointers needed
    {
        const ssd_shape s = shape(0, 100, 8, 64, 128, 2, SSD_DTYPE_BF16);
        const long before = launches();
        CHECK(ssd_chunk_scan_fwd(&s, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 256, nullptr,
                                 nullptr, nullptr, nullptr, 0, nullptr) == SSD_OK);
        CHECK(launches() == before);
    }
    // final_states may be the very buffer of initial_states
    {
        const ssd_shape s = shape(1, 300, 4, 32, 16, 1, SSD_DTYPE_F32);
        Args a = args_for(s, 64, f);
        a.init = a.fin;
        CHECK(fwd(s, 64, a) == SSD_OK);
    }
    // a valid decode step: one launch
    {
        const ssd_shape d1 = shape(4, 1, 8, 64, 128, 2, SSD_DTYPE_F32);
        const long c4 = g_launches[4];
        CHECK(ssd_decode_step(&d1, f(), f(), (const float *)f(), f(), f(), nullptr, (float *)f(), f(), nullptr,
                              nullptr) == SSD_OK);
        CHECK(g_launches[4] == c4 + 1);
    }
    for (int st = 0; st <= 6; ++st) CHECK(std::strlen(ssd_status_string((ssd_status)st)) > 1);
    CHECK(ssd_version() >= 200);
}

// Queries and (stub-launching) forward calls from many threads at once; every
// thread must see the single-threaded answers.
static void threads() {
    const ssd_shape shapes[] = {
        shape(2, 2048, 80, 64, 128, 1, SSD_DTYPE_BF16), shape(8, 4096, 80, 64, 128, 1, SSD_DTYPE_BF16),
        shape(1, 65536, 32, 64, 256, 1, SSD_DTYPE_BF16), shape(4, 16384, 64, 128, 256, 8, SSD_DTYPE_F32),
        shape(1, 256, 4, 32, 16, 1, SSD_DTYPE_F32)};
    const int64_t chunks[] = {256, 256, 256, 128, 64};
    size_t want_size[5];
    ssd_workspace_layout want_lay[5];
    ssd_plan want_plan[5];
    for (int i = 0; i < 5; ++i) {
        want_size[i] = ssd_chunk_scan_fwd_workspace_size(&shapes[i], chunks[i]);
        CHECK(ssd_chunk_scan_fwd_workspace_layout(&shapes[i], chunks[i], &want_lay[i]) == SSD_OK);
        CHECK(ssd_chunk_scan_fwd_default_plan(&shapes[i], chunks[i], &want_plan[i]) == SSD_OK);
    }
    std::atomic<int> bad{0};
    std::vector<std::thread> pool;
    for (int t = 0; t < 8; ++t)
        pool.emplace_back([&, t]() {
            Fake f;
            for (int it = 0; it < 300; ++it) {
                const int i = (it + t) % 5;
                ssd_workspace_layout lay;
                ssd_plan plan;
                if (ssd_chunk_scan_fwd_workspace_size(&shapes[i], chunks[i]) != want_size[i]) bad++;
                if (ssd_chunk_scan_fwd_workspace_layout(&shapes[i], chunks[i], &lay) != SSD_OK ||
                    std::memcmp(&lay, &want_lay[i], sizeof(lay)) != 0)
                    bad++;
                if (ssd_chunk_scan_fwd_default_plan(&shapes[i], chunks[i], &plan) != SSD_OK ||
                    std::memcmp(&plan, &want_plan[i], sizeof(plan)) != 0)
                    bad++;
                Args a = args_for(shapes[i], chunks[i], f);
                if (fwd(shapes[i], chunks[i], a) != SSD_OK) bad++;
            }
        });
    for (auto &th : pool) th.join();
    CHECK(bad == 0);
}

int main() {
    validation_paths();
    valid_calls();
    threads();
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
