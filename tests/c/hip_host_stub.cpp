// Host-only stand-ins for what libconvverify.so links from its device objects and the
// HIP runtime, so that the C-ABI layer (cv_api.cpp) can be built and run on a machine
// without a GPU under AddressSanitizer / UndefinedBehaviorSanitizer.  Test code only.
//
// Each kernel picker returns the address of a marker that encodes its arguments, and
// hipLaunchKernel records the launch (grid, block, LDS, the argument struct's bytes)
// instead of running anything, so a driver can check which kernel a call picked and
// with what geometry.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>

#include "cv_internal.h"

namespace {
// marker[k] for k = kernel code (see code_of): distinct addresses, never dereferenced
char g_marker[1 << 18];
}

extern "C" {
// What the last hipLaunchKernel call received.
struct stub_launch {
    int count;
    int code;             // kernel code of the function pointer (-1: not a marker)
    unsigned grid_x, block_x;
    size_t lds;
    unsigned char args[512];
};
stub_launch g_stub_launch;
hipError_t g_stub_launch_result = hipSuccess;
}

static const void *marker(int code) { return &g_marker[code]; }

// code: family (0 verify, 1 split, 2 restore, 3 prefill, 4 l2) in bits 14..16, the
// verify pickers' line-aligned, lean and split flags in bits 17, 13 and 12 (builds 2 and
// 1), the picker's other arguments in four 3-bit fields below
static int code_of(int family, int a, int b, int c, int d) {
    return family << 14 | (a & 7) << 9 | (b & 7) << 6 | (c & 7) << 3 | (d & 7);
}

namespace cvimpl {
#define CV_STUB_PICK(xb, sb, v, tm)                                                       \
    const void *pick_kernel_##xb##_##sb##_##v##_##tm(int d_conv, int tb, int build, int split) { \
        if (d_conv < 2 || d_conv > 4) return nullptr;                                     \
        int bucket = tb == 1 ? 0 : tb == 2 ? 1 : tb == 4 ? 2 : tb == 8 ? 3 : tb == 16 ? 4  \
                   : tb == 24 ? 5 : tb == 32 ? 6 : -1;                                    \
        if (bucket < 0) return nullptr;                                                   \
        /* the split build exists for the row layouts' buckets 8 and 16; other variants */ \
        /* take no split argument */                                                      \
        const bool rows = (v) == 1 || (v) == 2;                                           \
        if (split && rows && tb != 8 && tb != 16) return nullptr;                         \
        return marker(code_of(0, (xb) * 2 + (sb) / 2 - 3, (v) * 2 + (tm), d_conv, bucket) | \
                      (build == 1 ? 1 << 13 : 0) | (build == 2 ? 1 << 17 : 0) |          \
                      (split && rows ? 1 << 12 : 0));                                     \
    }
#define CV_STUB_PICKS(xb, sb) \
    CV_STUB_PICK(xb, sb, 0, 0) CV_STUB_PICK(xb, sb, 1, 0) CV_STUB_PICK(xb, sb, 2, 0) CV_STUB_PICK(xb, sb, 3, 0) \
    CV_STUB_PICK(xb, sb, 0, 1) CV_STUB_PICK(xb, sb, 1, 1) CV_STUB_PICK(xb, sb, 2, 1) CV_STUB_PICK(xb, sb, 3, 1)
CV_STUB_PICKS(4, 4)
CV_STUB_PICKS(2, 2)
CV_STUB_PICKS(2, 4)

const void *pick_restore(int state_bytes, int d_conv, int layout, int tm) {
    return marker(code_of(2, state_bytes, d_conv, layout, tm));
}
const void *pick_split(int x_bytes, int state_bytes, int d_conv, int tm) {
    return marker(code_of(1, x_bytes, state_bytes, d_conv, tm));
}
const void *pick_prefill(int x_bytes, int state_bytes, int d_conv, int tm) {
    return marker(code_of(3, x_bytes, state_bytes, d_conv, tm));
}
const void *pick_l2(int x_bytes) { return marker(code_of(4, x_bytes, 0, 0, 0)); }
}  // namespace cvimpl

extern "C" {
hipError_t hipLaunchKernel(const void *fn, dim3 grid, dim3 block, void **args, size_t lds,
                           hipStream_t stream) {
    (void)stream;
    g_stub_launch.count++;
    const char *p = static_cast<const char *>(fn);
    g_stub_launch.code = (p >= g_marker && p < g_marker + sizeof g_marker) ? (int)(p - g_marker) : -1;
    g_stub_launch.grid_x = grid.x;
    g_stub_launch.block_x = block.x;
    g_stub_launch.lds = lds;
    // every entry point passes one argument, its struct by pointer; its type follows
    // from the kernel family
    std::memset(g_stub_launch.args, 0, sizeof g_stub_launch.args);
    if (g_stub_launch.code >= 0) {
        const int family = (g_stub_launch.code >> 14) & 7;
        const size_t n = family <= 1 ? sizeof(cvimpl::KernelArgs)
                       : family == 2 ? sizeof(cvimpl::RestoreArgs)
                       : family == 3 ? sizeof(cvimpl::PrefillArgs) : sizeof(cvimpl::L2Args);
        static_assert(sizeof(cvimpl::KernelArgs) <= sizeof g_stub_launch.args, "args record");
        std::memcpy(g_stub_launch.args, args[0], n);
    }
    return g_stub_launch_result;
}

const char *hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "stub error"; }
}
