// The allocation-free forward (sffn_forward_noalloc in include/sffn.h): the
// decode-regime forward with its workspace in a file-scope device array
// instead of caller-provided memory, for callers that cannot allocate.
//
// `scratch` below is a device symbol: in host code its name is only a
// stand-in, never a device address. Each device's copy is at its own address,
// obtained once per device with hipGetSymbolAddress (with that device
// current) and kept in scratch_ptr; host code passes that pointer to the
// kernels, never the array's name.
#include <mutex>

#include "sffn_internal.h"

namespace sffn {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[SFFN_STATIC_SCRATCH_BYTES];

namespace {
struct DeviceScratch {
    void *ptr = nullptr;       // this device's copy of `scratch`
    int n_cu = 0;
    sffn_shape shape{};        // shape of the last forward on this device
    bool inited = false;       // its layout's control block and slots cleared
};
std::mutex scratch_mu;
DeviceScratch scratch_dev[kMaxDevices];
}  // namespace

}  // namespace sffn

using namespace sffn;

static bool same_shape(const sffn_shape &a, const sffn_shape &b)
{
    return a.d_model == b.d_model && a.d_ff == b.d_ff && a.rank == b.rank && a.max_tokens == b.max_tokens &&
           a.dtype == b.dtype;
}

extern "C" sffn_status sffn_forward_noalloc(const sffn_shape *shape, const void *x, int n_tokens,
                                            const sffn_weights *w, int mode, float tau, int k, float *y,
                                            int32_t *active_idx, int32_t *active_cnt, int32_t *union_cnt,
                                            float *debug_z, void *stream)
{
    // ---- validation: host only, nothing enqueued on failure ----
    if (!shape || !shape_ok(*shape)) return SFFN_ERR_INVALID_ARG;
    if (shape->max_tokens > kDecodeMaxTokens) return SFFN_ERR_UNSUPPORTED;
    const sffn_status v =
        forward_checks(*shape, x, n_tokens, w, mode, tau, k, y, active_idx, active_cnt, union_cnt, debug_z);
    if (v != SFFN_OK) return v;
    const Layout L = make_layout(*shape);
    if (L.total > (size_t)SFFN_STATIC_SCRATCH_BYTES) return SFFN_ERR_WORKSPACE;
    if (n_tokens == 0) return SFFN_OK;

    // ---- this device's scratch: its address and compute units, once ----
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SFFN_ERR_HIP;
    std::lock_guard<std::mutex> lock(scratch_mu);
    DeviceScratch &ds = scratch_dev[dev];
    sffn_ctx c{};
    if (!ds.ptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SFFN_ERR_HIP;
        if (device_setup(c) != hipSuccess) return SFFN_ERR_HIP;
        ds.ptr = p;
        ds.n_cu = c.n_cu;
    }
    // The array keeps the last forward's contents. A forward of another
    // shape lays the workspace out differently, so its control block and
    // slots are cleared first (as for a new handle).
    if (!same_shape(ds.shape, *shape)) {
        ds.shape = *shape;
        ds.inited = false;
    }
    c.shape = *shape;
    c.ws = static_cast<char *>(ds.ptr);
    c.ws_bytes = SFFN_STATIC_SCRATCH_BYTES;
    c.L = L;
    c.inited = ds.inited;
    c.n_cu = ds.n_cu;
    c.spin_max = kSpinMaxDefault;
    c.token_groups = 1;
    c.ev_start = c.ev_stop = nullptr;
    const sffn_status st = forward_enqueue(
        c, make_fwd(x, n_tokens, w, mode, tau, k, y, active_idx, active_cnt, union_cnt, debug_z, stream));
    ds.inited = c.inited;
    return st;
}
