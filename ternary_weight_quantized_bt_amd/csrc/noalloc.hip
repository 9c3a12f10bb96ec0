// noalloc.hip -- the per-layer driver for callers that cannot allocate
// device memory or hand in a workspace (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  It runs exactly the
// kernels of bt_layer_forward; the scratch they stage the quantized inputs
// in is a static device array that the library holds on every GPU it runs
// on until the process ends, instead of the caller's workspace.
//
// The array's name is a host-side stand-in, not a device address: host code
// uses only the address hipGetSymbolAddress returns for the current device,
// looked up once per device (with that device current) and kept.  Every call
// on a GPU shares that GPU's array, which keeps the last call's contents; the
// kernels overwrite everything they read from it before reading it, so
// nothing needs clearing.  Calls that overlap on one GPU race.

#include <stdio.h>

#include <mutex>

#include "internal.hpp"

static __device__ __align__(256) uint8_t scratch[BT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // the array's device address per device (null: not looked up)

// Device address of the current device's copy of `scratch`.
hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

}  // namespace

extern "C" bt_status bt_layer_forward_noalloc(const bt_layer *layer, const bt_layer_io *io,
                                              bt_stream stream) {
    const char *fn = "bt_layer_forward_noalloc";
    size_t need = 0;
    const bt_status st = bt::layer_check(layer, io, fn, &need);
    if (st != BT_OK || io->N == 0) return st;
    if (need > (size_t)BT_NOALLOC_SCRATCH_BYTES) {
        char msg[256];
        snprintf(msg, sizeof msg,
                 "%s: %lld tokens of this layer need %zu bytes of scratch, more than the "
                 "%u bytes of static scratch (use bt_layer_forward with a workspace)",
                 fn, (long long)io->N, need, (unsigned)BT_NOALLOC_SCRATCH_BYTES);
        return bt::fail_with(BT_ERR_WORKSPACE, msg);
    }
    void *p = nullptr;
    const hipError_t e = scratch_address(&p);
    if (e != hipSuccess) {
        char msg[256];
        snprintf(msg, sizeof msg, "%s: looking up the static scratch: %s", fn,
                 hipGetErrorString(e));
        return bt::fail_with(BT_ERR_HIP, msg);
    }
    return bt::layer_forward(layer, io, p, (size_t)BT_NOALLOC_SCRATCH_BYTES, stream, fn);
}
