// Drives the C-ABI layer of libdcnv4 (argument checks, output sizes, tile
// planning, launch splitting) over a seeded sweep of valid and invalid
// calls, against the host-only launch stand-ins of host_fakes.cpp.  Built
// with AddressSanitizer and UndefinedBehaviorSanitizer by the test suite;
// prints "ok <cases>" and exits 0 when every call returned a documented
// status and every launch stayed inside the caller's tensors.
#include "dcnv4.h"
#include "flash_deform_attn.h"

#include "fakes.h"

#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;

uint32_t rnd()
{
    // splitmix64
    uint64_t z = (g_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return (uint32_t)((z ^ (z >> 31)) >> 32);
}

int pick(const int *v, int n)
{
    return v[rnd() % n];
}

int range(int lo, int hi)
{
    return lo + (int)(rnd() % (uint32_t)(hi - lo + 1));
}

long g_cases = 0;
long g_accepted = 0;   // calls that returned DCNV4_OK

[[noreturn]] void fail(const char *what, int st)
{
    std::fprintf(stderr, "case %ld: %s (status %d)\n", g_cases, what, st);
    std::exit(1);
}

bool documented(int st)
{
    return st <= 0 && st >= DCNV4_ERR_HIP;
}

// Fake device addresses: never dereferenced by the C-ABI layer; each tensor
// gets its own 256-byte aligned range.
uintptr_t g_next = 0x100000000000ull;

void *tensor(int64_t bytes)
{
    void *p = reinterpret_cast<void *>(g_next);
    g_next += ((uintptr_t)(bytes > 0 ? bytes : 1) + 255) / 256 * 256 + 256;
    if (g_next > 0x700000000000ull)
        g_next = 0x100000000000ull;
    fake::add_range(p, bytes);
    return p;
}

struct Conv {
    int N, H, W, kh, kw, sh, sw, ph, pw, dh, dw, G, Cg, rc, P, sm, dtype;
    float scale;
};

int es_of(int dtype)
{
    return dtype == DCNV4_FP32 ? 4 : 2;
}

// One forward and one backward call; checks statuses and image counts.
void run_conv(const Conv &c, bool expect_ok)
{
    int Ho = 0, Wo = 0;
    const int st_sz = dcnv4_output_size(c.H, c.W, c.kh, c.kw, c.sh, c.sw, c.ph, c.pw, c.dh, c.dw, &Ho, &Wo);
    if (!documented(st_sz))
        fail("output_size status", st_sz);
    const int64_t es = (c.dtype >= 0 && c.dtype <= 2) ? es_of(c.dtype) : 4;
    const int64_t C = (int64_t)c.G * c.Cg;
    const bool sized = st_sz == DCNV4_OK && c.N >= 0 && C > 0 && c.P > 0;
    // tensors are registered only when their sizes are meaningful; beyond
    // 2^46 bytes the call must refuse them anyway
    auto bytes = [&](double a, double b, double cc, double d) -> int64_t {
        if (!sized)
            return 16;
        const double v = a * b * cc * d;
        return v > 7.0e13 ? 16 : (int64_t)v;
    };
    for (int backward = 0; backward < 2; ++backward) {
        ++g_cases;
        fake::reset();
        const int64_t nv = bytes(c.N, c.H, c.W, (double)C * es), nom = bytes(c.N, Ho, Wo, (double)c.P * es),
                      no = bytes(c.N, Ho, Wo, (double)C * es), ngv = bytes(c.N, c.H, c.W, (double)C * 4);
        void *v = tensor(nv), *om = tensor(nom), *o = tensor(no);
        int st;
        if (!backward) {
            st = dcnv4_forward_ex(v, om, o, c.N, c.H, c.W, c.kh, c.kw, c.sh, c.sw, c.ph, c.pw, c.dh, c.dw, c.G, c.Cg,
                                  c.scale, c.rc, c.P, c.sm, c.dtype, nullptr);
        } else {
            void *gv = tensor(ngv), *gom = tensor(nom);
            st = dcnv4_backward_ex(v, om, o, gv, gom, c.N, c.H, c.W, c.kh, c.kw, c.sh, c.sw, c.ph, c.pw, c.dh, c.dw,
                                   c.G, c.Cg, c.scale, c.rc, c.P, c.sm, c.dtype, nullptr);
        }
        if (!documented(st) || st == DCNV4_ERR_HIP)
            fail("conv status", st);
        g_accepted += st == DCNV4_OK;
        if (st == DCNV4_OK && fake::g_images != (c.N > 0 ? c.N : 0))
            fail("images launched != N", (int)fake::g_images);
        if (st != DCNV4_OK && fake::g_launches != 0)
            fail("launch before a failing check", st);
        if (expect_ok && st != DCNV4_OK)
            fail("expected DCNV4_OK", st);
    }
}

const int kCg[] = {1, 4, 8, 12, 16, 24, 32, 48, 64, 128, 256};
const int kG[] = {1, 2, 3, 4, 5, 8, 16, 32, 64};
const int kN[] = {0, 1, 1, 2, 3, 5, 8, 64};
const int kK[] = {1, 3, 3, 3, 5, 7, 2, 4};
const int kFN[] = {0, 1, 2, 4, 32};
const int kFQ[] = {0, 1, 7, 300, 5000};
const int kFM[] = {1, 2, 8};
const int kFD[] = {4, 8, 16, 32, 64, 128};

void sweep_conv(int cases)
{
    for (int i = 0; i < cases; ++i) {
        Conv c;
        const bool big = rnd() % 16 == 0;
        c.N = pick(kN, 8);
        c.H = big ? range(1, 3000) : range(1, 80);
        c.W = big ? range(1, 3000) : range(1, 80);
        c.kh = pick(kK, 8);
        c.kw = rnd() % 4 ? c.kh : pick(kK + 3, 3);
        c.sh = range(1, 3);
        c.sw = rnd() % 2 ? c.sh : range(1, 3);
        c.ph = range(0, 4);
        c.pw = range(0, 4);
        c.dh = range(1, 3);
        c.dw = range(1, 3);
        c.G = pick(kG, 9);
        c.Cg = pick(kCg, 11);
        c.rc = rnd() % 4 == 0;
        c.sm = rnd() % 4 == 0;
        c.dtype = range(0, 2);
        c.scale = (float)(rnd() % 1000) / 250.0f;
        const int om = dcnv4_om_channels(c.G, c.kh, c.kw, c.rc);
        c.P = om > 0 ? om + 8 * (int)(rnd() % 2) : 8;
        // occasional invalid arguments
        switch (rnd() % 24) {
        case 0: c.N = -1; break;
        case 1: c.sh = 0; break;
        case 2: c.ph = -1; break;
        case 3: c.dtype = 7; break;
        case 4: c.P = c.P - 4; break;
        case 5: c.sm = 2; break;
        case 6: c.rc = 2; break;
        case 7: c.G = 0; break;
        default: break;
        }
        run_conv(c, false);
    }
}

void conv_edges()
{
    // ordinary shapes that must be accepted
    Conv ok[] = {
        {64, 56, 56, 3, 3, 1, 1, 1, 1, 1, 1, 4, 16, 0, 112, 0, DCNV4_FP32, 1.0f},
        {64, 56, 56, 3, 3, 1, 1, 1, 1, 1, 1, 4, 16, 0, 112, 0, DCNV4_FP16, 1.0f},
        {64, 7, 7, 3, 3, 1, 1, 1, 1, 1, 1, 32, 16, 0, 864, 0, DCNV4_FP16, 1.0f},
        {1, 270, 480, 3, 3, 1, 1, 1, 1, 1, 1, 16, 16, 0, 432, 0, DCNV4_BF16, 1.0f},
        {1, 270, 480, 3, 3, 1, 1, 1, 1, 1, 1, 16, 16, 1, 384, 0, DCNV4_BF16, 1.0f},
        {2, 14, 14, 5, 5, 1, 1, 2, 2, 1, 1, 4, 16, 0, 304, 1, DCNV4_FP32, 0.5f},
        {4096, 56, 56, 3, 3, 1, 1, 1, 1, 1, 1, 4, 16, 0, 112, 0, DCNV4_FP32, 1.0f},   // split launches
        {1, 1, 1, 1, 1, 1, 1, 0, 0, 1, 1, 1, 4, 0, 8, 0, DCNV4_FP32, 1.0f},
    };
    for (const Conv &c : ok)
        run_conv(c, true);
    // sizes at the edges of the index range: a documented refusal, no UB
    Conv bad[] = {
        {1, 30000, 30000, 3, 3, 1, 1, 1, 1, 1, 1, 64, 64, 0, 1728, 0, DCNV4_FP32, 1.0f},
        {INT_MAX, 56, 56, 3, 3, 1, 1, 1, 1, 1, 1, 4, 16, 0, 112, 0, DCNV4_FP32, 1.0f},
        {1, INT_MAX, INT_MAX, 3, 3, 1, 1, 1, 1, 1, 1, 1, 4, 0, 32, 0, DCNV4_FP32, 1.0f},
        {1, 8, 8, INT_MAX, INT_MAX, 1, 1, 1, 1, 1, 1, 1, 4, 0, 8, 0, DCNV4_FP32, 1.0f},
        {1, 8, 8, 3, 3, INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, INT_MAX, 1, 4, 0, 16, 0, DCNV4_FP32, 1.0f},
        {1, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1, INT_MAX, INT_MAX, 0, 16, 0, DCNV4_FP32, 1.0f},
        {1, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1, 65536, 65536, 0, INT_MAX - 7, 0, DCNV4_FP32, 1.0f},
        {1, 8, 8, 3, 3, 1, 1, 1, 1, 1, 1, 4, 16, 0, INT_MAX, 0, DCNV4_FP32, 1.0f},
    };
    for (const Conv &c : bad)
        run_conv(c, false);
    for (int v : {INT_MIN, -1, 0, 1, 3, 65535, INT_MAX}) {
        ++g_cases;
        const int st = dcnv4_om_channels(v, v, v, 0);
        if (st < 0 && !documented(st))
            fail("om_channels status", st);
        int Ho, Wo;
        const int s2 = dcnv4_output_size(v, v, v, v, v, v, v, v, v, v, &Ho, &Wo);
        if (!documented(s2))
            fail("output_size status", s2);
    }
    // pointer errors of an otherwise valid call
    ++g_cases;
    fake::reset();
    void *v = tensor(56 * 56 * 64 * 4), *om = tensor(56 * 56 * 112 * 4), *o = tensor(56 * 56 * 64 * 4);
    if (dcnv4_forward(nullptr, om, o, 1, 56, 56, 3, 3, 1, 1, 1, 1, 1, 1, 4, 16, 1.0f, 0, 112, DCNV4_FP32, nullptr) !=
        DCNV4_ERR_NULL)
        fail("NULL value accepted", 0);
    if (dcnv4_forward(static_cast<char *>(v) + 4, om, o, 1, 56, 56, 3, 3, 1, 1, 1, 1, 1, 1, 4, 16, 1.0f, 0, 112,
                      DCNV4_FP32, nullptr) != DCNV4_ERR_ALIGN)
        fail("misaligned value accepted", 0);
    if (dcnv4_forward(v, om, static_cast<char *>(v) + 1024, 1, 56, 56, 3, 3, 1, 1, 1, 1, 1, 1, 4, 16, 1.0f, 0, 112,
                      DCNV4_FP32, nullptr) != DCNV4_ERR_PARAM)
        fail("overlap accepted", 0);
    if (fake::g_launches != 0)
        fail("launch on a refused call", 0);
    for (int st = 1; st >= -9; --st)
        if (!dcnv4_status_string(st))
            fail("status string", st);
}

// ---- flash deformable attention ----

void run_fda(int N, int L, const int *shapes, int Q, int M, int D, int K, int P, int dtype, bool expect_ok)
{
    int64_t S = 0;
    for (int l = 0; l < L; ++l)
        S += (int64_t)shapes[2 * l] * shapes[2 * l + 1];
    const int Si = S > INT_MAX ? INT_MAX : (int)S;
    const int64_t es = dtype == DCNV4_FP32 ? 4 : 2;
    auto bytes = [&](double a, double b, double c) -> int64_t {
        const double v = (N > 0 ? N : 1) * a * b * c;
        return v > 7.0e13 || v < 0 ? 16 : (int64_t)v;
    };
    for (int mode = 0; mode < 4; ++mode) {   // forward, backward with / without workspace, no-alloc
        ++g_cases;
        fake::reset();
        void *v = tensor(bytes(Si, M, (double)D * es)), *loc = tensor(bytes(Q, M, (double)P * es)),
             *o = tensor(bytes(Q, M, (double)D * es));
        int st;
        if (mode == 0) {
            st = flash_deform_attn_forward(v, shapes, L, loc, o, N, Si, Q, M, D, K, P, dtype, nullptr);
        } else {
            void *gv = tensor(bytes(Si, M, (double)D * 4)), *gl = tensor(bytes(Q, M, (double)P * es));
            if (mode == 3) {
                fake::add_range(fake::noalloc_base(), FLASH_DEFORM_ATTN_NOALLOC_SCRATCH_BYTES);
                st = flash_deform_attn_backward_noalloc(v, shapes, L, loc, o, gv, gl, N, Si, Q, M, D, K, P, dtype,
                                                        nullptr);
            } else {
                size_t ws = 0;
                const int sw = flash_deform_attn_backward_workspace(shapes, L, N, Si, Q, M, D, K, P, dtype, &ws);
                if (!documented(sw))
                    fail("workspace status", sw);
                void *w = mode == 1 && sw == DCNV4_OK && ws > 0 && ws < (size_t)7e13 ? tensor((int64_t)ws) : nullptr;
                st = flash_deform_attn_backward(v, shapes, L, loc, o, gv, gl, w, w ? ws : 0, N, Si, Q, M, D, K, P,
                                                dtype, nullptr);
            }
        }
        if (!documented(st) || st == DCNV4_ERR_HIP)
            fail("fda status", st);
        const long want = (N > 0 && Q > 0) ? N : 0;
        g_accepted += st == DCNV4_OK;
        if (st == DCNV4_OK && fake::g_images != want)
            fail("fda images launched != N", (int)fake::g_images);
        if (st != DCNV4_OK && fake::g_launches != 0)
            fail("fda launch before a failing check", st);
        if (expect_ok && st != DCNV4_OK && !(mode == 3 && st == DCNV4_ERR_UNSUPPORTED))
            fail("fda expected DCNV4_OK", st);
    }
}

void sweep_fda(int cases)
{
    int shapes[2 * 6];
    for (int i = 0; i < cases; ++i) {
        const int L = range(1, 5);
        const bool big = rnd() % 8 == 0;
        for (int l = 0; l < L; ++l) {
            shapes[2 * l] = big ? range(1, 400) : range(1, 40);
            shapes[2 * l + 1] = big ? range(1, 400) : range(1, 40);
        }
        const int N = pick(kFN, 5);
        const int Q = pick(kFQ, 5);
        const int M = pick(kFM, 3);
        const int D = pick(kFD, 6);
        const int K = range(1, 8);
        const int dtype = range(0, 2);
        const int P = (3 * L * K + 7) / 8 * 8 + 8 * (int)(rnd() % 2) - (rnd() % 16 == 0 ? 4 : 0);
        run_fda(N, L, shapes, Q, M, D, K, P, dtype, false);
    }
    const int s4[] = {100, 160, 50, 80, 25, 40, 13, 20};
    run_fda(2, 4, s4, 900, 8, 32, 4, 48, DCNV4_FP32, true);
    run_fda(64, 4, s4, 900, 8, 32, 4, 48, DCNV4_BF16, true);   // split launches
    const int huge[] = {46341, 46341};
    run_fda(1, 1, huge, 10, 1, 8, 1, 8, DCNV4_FP32, false);
}

}  // namespace

int main()
{
    conv_edges();
    sweep_conv(4000);
    sweep_fda(1500);
    std::printf("ok %ld calls, %ld accepted\n", g_cases, g_accepted);
    return 0;
}
