// Host-only stand-ins for the HIP runtime calls and kernel launches that
// the C-ABI layer (dcnv4_api.cpp, fdattn_api.cpp) makes, so that its
// argument checks, planning and launch splitting can run on a machine
// without a GPU under AddressSanitizer / UndefinedBehaviorSanitizer.
//
// Every "launch" checks, instead of enqueueing a kernel, that the plan it is
// given is one a kernel could run (threads, LDS, tiles covering the output)
// and that every byte range it would touch lies inside one of the tensors
// the test registered for the current call; it counts the images.
#include "dcnv4_internal.h"
#include "fdattn_internal.h"

#include "fakes.h"

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace fake {

struct Range {
    uintptr_t base;
    int64_t bytes;
};

static std::vector<Range> g_ranges;
long g_images = 0;
long g_launches = 0;

void reset()
{
    g_ranges.clear();
    g_images = 0;
    g_launches = 0;
}

void add_range(const void *base, int64_t bytes)
{
    g_ranges.push_back({reinterpret_cast<uintptr_t>(base), bytes});
}

[[noreturn]] static void fail(const char *what)
{
    std::fprintf(stderr, "host fake: %s\n", what);
    std::abort();
}

// [p, p + bytes) lies inside one registered tensor
static void inside(const void *p, int64_t bytes, const char *what)
{
    if (bytes < 0)
        fail(what);
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    for (const Range &r : g_ranges)
        if (a >= r.base && a + (uintptr_t)bytes <= r.base + (uintptr_t)r.bytes)
            return;
    fail(what);
}

void *noalloc_base()
{
    return reinterpret_cast<void *>(uintptr_t(0x7e0000000000));
}

static void count(int n)
{
    if (n < 1)
        fail("launch of no images");
    g_images += n;
    g_launches += 1;
}

}  // namespace fake

// ---- HIP runtime calls made by the C-ABI layer ----
extern "C" {
hipError_t hipGetDevice(int *dev)
{
    *dev = 0;
    return hipSuccess;
}
hipError_t hipFuncSetAttribute(const void *, hipFuncAttribute, int value)
{
    return value <= 160 * 1024 ? hipSuccess : hipErrorInvalidValue;
}
const char *hipGetErrorName(hipError_t)
{
    return "hipErrorFake";
}
const char *hipGetErrorString(hipError_t)
{
    return "fake error";
}
}

namespace dcnv4 {

static void check_problem(const Problem &p)
{
    if (p.N < 1 || p.H < 1 || p.W < 1 || p.Ho < 1 || p.Wo < 1 || p.G < 1 || p.Cg < 1 || p.K < 1 ||
        p.P < 3 * p.G * p.K || p.C != p.G * p.Cg)
        fake::fail("problem");
}

static void check_extents(const Problem &p, const void *value, const void *om, const void *out, int out_elem,
                          const void *go, const void *gv, const void *gom)
{
    const int64_t es = p.elem;
    fake::inside(value, (int64_t)p.N * p.H * p.W * p.C * es, "value extent");
    fake::inside(om, (int64_t)p.N * p.Ho * p.Wo * p.P * es, "offset_mask extent");
    if (out)
        fake::inside(out, (int64_t)p.N * p.Ho * p.Wo * p.C * out_elem, "output extent");
    if (go)
        fake::inside(go, (int64_t)p.N * p.Ho * p.Wo * p.C * es, "grad_output extent");
    if (gv)
        fake::inside(gv, (int64_t)p.N * p.H * p.W * p.C * 4, "grad_value extent");
    if (gom)
        fake::inside(gom, (int64_t)p.N * p.Ho * p.Wo * p.P * es, "grad_offset_mask extent");
    // a launch's buffers must fit 31-bit byte offsets
    const int64_t lim = 0x7fffffff;
    if ((int64_t)p.N * p.H * p.W * p.C * es > lim || (int64_t)p.N * p.Ho * p.Wo * p.P * es > lim ||
        (int64_t)p.N * p.Ho * p.Wo * p.C * es > lim || (gv && (int64_t)p.N * p.H * p.W * p.C * 4 > lim) ||
        (gom && (int64_t)p.N * p.Ho * p.Wo * p.P * es > lim))
        fake::fail("launch exceeds 31-bit offsets");
}

static void check_general(const Problem &p, const Plan &plan)
{
    if (plan.threads < 1 || plan.threads > 1024 || plan.lds_bytes < 0 || plan.lds_bytes > 160 * 1024 ||
        plan.dp < 1 || plan.lanes * plan.dp != p.Cg || plan.pix_per_block < 1)
        fake::fail("general plan");
}

static void check_tiled(const Problem &p, const TilePlan &tp, bool backward)
{
    if (tp.threads < 64 || tp.threads > 1024 || tp.threads % 64 || tp.lds_bytes < 1 || tp.lds_bytes > 160 * 1024 ||
        tp.th < 1 || tp.tw < 1 || (int64_t)tp.tiles_y * tp.th < p.Ho || (int64_t)tp.tiles_x * tp.tw < p.Wo ||
        tp.R < 0 || tp.rh < 2 || tp.rw < 2 || tp.lanes * tp.dp * 1 < 1)
        fake::fail("tile plan");
    if (backward && (tp.splat_lds_bytes < 1 || tp.splat_lds_bytes > 160 * 1024 || tp.ch < 1 || tp.cw < 1 ||
                     (int64_t)tp.ctiles_y * tp.ch < p.H || (int64_t)tp.ctiles_x * tp.cw < p.W))
        fake::fail("cell plan");
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t)
{
    fake::inside(p, (int64_t)bytes, "zero extent");
    return hipSuccess;
}

hipError_t launch_forward_general(const Problem &p, const Plan &plan, const void *value, const void *om, void *out,
                                  hipStream_t)
{
    check_problem(p);
    check_general(p, plan);
    check_extents(p, value, om, out, p.elem, nullptr, nullptr, nullptr);
    fake::count(p.N);
    return hipSuccess;
}

hipError_t launch_backward_general(const Problem &p, const Plan &plan, const void *value, const void *om,
                                   const void *go, void *gv, void *gom, hipStream_t)
{
    check_problem(p);
    check_general(p, plan);
    check_extents(p, value, om, nullptr, 0, go, gv, gom);
    fake::count(p.N);
    return hipSuccess;
}

hipError_t launch_forward_tiled(const Problem &p, const TilePlan &tp, const void *value, const void *om, void *out,
                                hipStream_t)
{
    check_problem(p);
    check_tiled(p, tp, false);
    check_extents(p, value, om, out, p.elem, nullptr, nullptr, nullptr);
    fake::count(p.N);
    return hipSuccess;
}

hipError_t launch_backward_tiled(const Problem &p, const TilePlan &tp, const void *value, const void *om,
                                 const void *go, void *gv, void *gom, hipStream_t)
{
    check_problem(p);
    check_tiled(p, tp, true);
    check_extents(p, value, om, nullptr, 0, go, gv, gom);
    fake::count(p.N);
    return hipSuccess;
}

}  // namespace dcnv4

namespace fdattn {

// Stand-in size: the sort's real layout lives with its kernels; any size
// that grows with the launch exercises the splitting logic the same way.
size_t workspace_bytes(const Problem &p)
{
    return ((size_t)p.N * p.M * p.S * 8 + (size_t)p.N * p.M * p.Q * p.L * p.K * 36 + 255) / 256 * 256;
}

hipError_t noalloc_scratch(void **ptr)
{
    // a host address standing for the device array; its extent is
    // registered by the test like a caller's workspace
    *ptr = fake::noalloc_base();
    return hipSuccess;
}

static void check_fda(const Problem &p, const void *value, const void *loc, const void *out_or_go)
{
    if (p.N < 1 || p.Q < 1 || p.M < 1 || p.D < 1 || p.K < 1 || p.L < 1 || p.P < 3 * p.L * p.K)
        fake::fail("fda problem");
    const int64_t es = p.elem;
    fake::inside(value, (int64_t)p.N * p.S * p.M * p.D * es, "fda value extent");
    fake::inside(loc, (int64_t)p.N * p.Q * p.M * p.P * es, "fda loc_attn extent");
    fake::inside(out_or_go, (int64_t)p.N * p.Q * p.M * p.D * es, "fda output extent");
}

hipError_t launch_forward(const Problem &p, const void *value, const void *loc, void *out, hipStream_t)
{
    check_fda(p, value, loc, out);
    fake::count(p.N);
    return hipSuccess;
}

hipError_t launch_backward(const Problem &p, const void *value, const void *loc, const void *go, float *gv,
                           void *gloc, void *workspace, hipStream_t)
{
    check_fda(p, value, loc, go);
    fake::inside(gv, (int64_t)p.N * p.S * p.M * p.D * 4, "fda grad_value extent");
    fake::inside(gloc, (int64_t)p.N * p.Q * p.M * p.P * p.elem, "fda grad_loc_attn extent");
    if (workspace)
        fake::inside(workspace, (int64_t)workspace_bytes(p), "fda workspace extent");
    fake::count(p.N);
    return hipSuccess;
}

}  // namespace fdattn
