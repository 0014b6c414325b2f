// ttt_linear_fwd for callers that cannot allocate (code under graph capture,
// tight serving loops, harnesses that forbid allocation): the same kernels as
// ttt_linear_fwd, with the scratch the state scan needs (the per-segment
// affine summaries and, for in-place calls, a copy of w_init) held in a
// file-scope device array instead of a caller workspace.
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Its device address is taken once per device with
// hipGetSymbolAddress (the array's name in host code is only a stand-in, not
// a device address) and that address is what the kernels receive.  Every call
// on a device shares the array: calls that overlap on one device (different
// streams, no ordering between them) race on it.  The scan writes every byte
// of scratch it later reads within the same call, so nothing needs clearing
// between calls.
#include "../../include/ttt.h"
#include "ttt_internal.h"

#include <hip/hip_runtime.h>
#include <mutex>
#include <stdint.h>

namespace {

constexpr size_t SCRATCH_BYTES = (size_t)64 << 20;   // stated maximum (64 MiB per device)
constexpr int MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

void *g_scratch_ptr[MAX_DEVICES];
std::once_flag g_scratch_once[MAX_DEVICES];
hipError_t g_scratch_err[MAX_DEVICES];

// Device address of this device's copy of `scratch` (the current device must
// be `dev`), looked up on the first call on that device.
void *scratch_ptr(int dev, hipError_t *err)
{
    std::call_once(g_scratch_once[dev], [dev]() {
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_err[dev] = e;
        g_scratch_ptr[dev] = (e == hipSuccess) ? p : nullptr;
    });
    *err = g_scratch_err[dev];
    return g_scratch_ptr[dev];
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" size_t ttt_linear_noalloc_max_scratch_bytes(void) { return SCRATCH_BYTES; }

extern "C" ttt_status ttt_linear_fwd_noalloc(const void *q, const void *k, const void *v, int dtype,
                                             const float *eta, const float *w_init, void *out,
                                             float *w_final, int B, int H, int Tq, int Tkv, int d,
                                             int chunk, int loss, int order, void *stream)
{
    // the same argument checks as ttt_linear_fwd (its workspace query answers
    // 0 for anything invalid or unsupported; the call itself says which)
    const size_t need =
        ttt_linear_workspace_bytes(B, H, Tq, Tkv, d, chunk, loss, order, dtype);
    if (need == 0) {
        // no scratch needed, or invalid/unsupported arguments: ttt_linear_fwd
        // validates and runs (with no workspace) or reports the error
        return ttt_linear_fwd(q, k, v, dtype, eta, w_init, out, w_final, B, H, Tq, Tkv, d, chunk,
                              loss, order, nullptr, 0, stream);
    }
    if (need > SCRATCH_BYTES) return TTT_EWORKSPACE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return TTT_EHIP;
    if (dev >= MAX_DEVICES) return TTT_EUNSUPPORTED;
    hipError_t err = hipSuccess;
    void *ws = scratch_ptr(dev, &err);
    if (err != hipSuccess || !ws || !aligned16(ws)) return TTT_EHIP;
    return ttt_linear_fwd(q, k, v, dtype, eta, w_init, out, w_final, B, H, Tq, Tkv, d, chunk, loss,
                          order, ws, SCRATCH_BYTES, stream);
}
