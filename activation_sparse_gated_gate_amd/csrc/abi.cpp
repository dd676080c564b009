// C ABI of the sparse gated-FFN forward: argument validation, workspace
// layout, handle lifetime and dispatch to the decode (GEMV) or batched (MFMA)
// kernels. Every check runs on the host before anything is enqueued; the
// declarations and their contracts are in include/sffn.h.
#include <cmath>
#include <cstring>
#include <new>

#include "sffn_internal.h"

namespace sffn {

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool shape_ok(const sffn_shape &s)
{
    if (s.d_model <= 0 || s.d_model % 8 != 0 || s.d_model > 65536) return false;
    if (s.d_ff < 1 || s.d_ff > kMaxDff) return false;
    if (s.rank < 0 || s.rank % 8 != 0 || s.rank > 16384) return false;
    if (s.max_tokens < 1 || s.max_tokens > 65536) return false;
    if (s.dtype != SFFN_F32 && s.dtype != SFFN_BF16) return false;
    return true;
}

Layout make_layout(const sffn_shape &s)
{
    Layout L{};
    const size_t F = (size_t)s.d_ff, d = (size_t)s.d_model, r = (size_t)s.rank;
    const size_t T = (size_t)s.max_tokens;
    const bool batched = s.max_tokens > kDecodeMaxTokens;
    L.words = (int)((F + 31) / 32);
    L.ntp = kDecodeMaxTokens;
    const size_t ntp = (size_t)L.ntp;
    const size_t rows = batched ? T : ntp;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + bytes);
        return at;
    };
    L.ctrl = take((size_t)kCtrlInts * 4);
    L.act = take(rows * F);
    const size_t FP = (F + 7) / 8 * 8;  // bf16 rows padded to 16 bytes
    L.gsel = take(batched ? (ntp * F * 4 > T * F * 2 ? ntp * F * 4 : T * F * 2) : ntp * F * 4);
    L.uidx = take(F * 4);
    L.hbuf = take(batched ? (F * ntp * 4 > T * FP * 2 ? F * ntp * 4 : T * FP * 2) : F * ntp * 4);
    L.any = take(F);
    L.part_words = (size_t)kDownGroupsMax * ntp * d;
    L.part = take(L.part_words * 4);
    L.tvec = take(r ? ntp * r * 4 : 0);
    L.keys = take(batched ? T * F * 4 : 0);
    L.ubits = take((size_t)L.words * 4);
    // room for every split a forward of up to T tokens takes, at least 16
    // splits of 64 tokens (forwards smaller than the handle's maximum)
    const size_t prow = T < 512 ? (size_t)splits_max((int)T) * T : 0, pmin = 16 * (T < 64 ? T : 64);
    L.bpart_rows = batched ? (int)(prow > pmin ? prow : pmin) : 0;
    L.bpart = take((size_t)L.bpart_rows * (F > d ? F : d) * 4);
    L.thr = take(rows * 8);
    L.total = off;
    return L;
}

}  // namespace sffn

using namespace sffn;

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
static bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

extern "C" {

size_t sffn_workspace_bytes(const sffn_shape *shape)
{
    if (!shape || !shape_ok(*shape)) return 0;
    return make_layout(*shape).total;
}

sffn_status sffn_create(const sffn_shape *shape, void *workspace, size_t workspace_bytes,
                        sffn_handle *out)
{
    if (!out) return SFFN_ERR_INVALID_ARG;
    *out = nullptr;
    if (!shape || !shape_ok(*shape)) return SFFN_ERR_INVALID_ARG;
    Layout L = make_layout(*shape);
    if (!workspace || ((uintptr_t)workspace & 255u) != 0 || workspace_bytes < L.total)
        return SFFN_ERR_WORKSPACE;
    sffn_ctx *c = new (std::nothrow) sffn_ctx();
    if (!c) return SFFN_ERR_INVALID_ARG;
    c->shape = *shape;
    c->ws = static_cast<char *>(workspace);
    c->ws_bytes = workspace_bytes;
    c->L = L;
    c->inited = false;
    c->n_cu = 0;
    c->lds_max = 0;
    c->ev_start = c->ev_stop = nullptr;
    *out = c;
    return SFFN_OK;
}

sffn_status sffn_destroy(sffn_handle handle)
{
    if (!handle) return SFFN_ERR_INVALID_ARG;
    delete handle;
    return SFFN_OK;
}

sffn_status sffn_set_profile_events(sffn_handle handle, void *ev_start, void *ev_stop)
{
    if (!handle) return SFFN_ERR_INVALID_ARG;
    if ((ev_start == nullptr) != (ev_stop == nullptr)) return SFFN_ERR_INVALID_ARG;
    handle->ev_start = ev_start;
    handle->ev_stop = ev_stop;
    return SFFN_OK;
}

const char *sffn_status_string(int status)
{
    switch (status) {
    case SFFN_OK: return "SFFN_OK";
    case SFFN_ERR_INVALID_ARG: return "SFFN_ERR_INVALID_ARG";
    case SFFN_ERR_UNSUPPORTED: return "SFFN_ERR_UNSUPPORTED";
    case SFFN_ERR_HIP: return "SFFN_ERR_HIP";
    case SFFN_ERR_WORKSPACE: return "SFFN_ERR_WORKSPACE";
    default: return "SFFN_ERR_UNKNOWN";
    }
}

sffn_status sffn_forward(sffn_handle handle, const void *x, int n_tokens, const sffn_weights *w,
                         int mode, float tau, int k, float *y, int32_t *active_idx,
                         int32_t *active_cnt, int32_t *union_cnt, float *debug_z, void *stream)
{
    // ---- validation: host only, nothing enqueued on failure ----
    if (!handle || !w) return SFFN_ERR_INVALID_ARG;
    const sffn_shape &s = handle->shape;
    if (n_tokens < 0 || n_tokens > s.max_tokens) return SFFN_ERR_INVALID_ARG;
    if (mode < SFFN_THRESHOLD || mode > SFFN_TOPP) return SFFN_ERR_INVALID_ARG;
    if (!x || !y || !aligned16(x) || !aligned16(y)) return SFFN_ERR_INVALID_ARG;
    if (!w->w_up || !w->w_down || !aligned16(w->w_up) || !aligned16(w->w_down))
        return SFFN_ERR_INVALID_ARG;
    if (mode == SFFN_LOPA) {
        if (s.rank <= 0) return SFFN_ERR_INVALID_ARG;
        if (!w->lopa_a || !w->lopa_b || !aligned16(w->lopa_a) || !aligned16(w->lopa_b))
            return SFFN_ERR_INVALID_ARG;
    } else {
        if (!w->w_gate || !aligned16(w->w_gate)) return SFFN_ERR_INVALID_ARG;
    }
    if (mode == SFFN_TOPK && (k < 1 || k > s.d_ff)) return SFFN_ERR_INVALID_ARG;
    if (mode != SFFN_TOPK && mode != SFFN_TOPK_2_8 && std::isnan(tau)) return SFFN_ERR_INVALID_ARG;
    if (mode == SFFN_TOPP && !(tau > 0.f && tau <= 1.f)) return SFFN_ERR_INVALID_ARG;
    if ((active_idx && !aligned4(active_idx)) || (active_cnt && !aligned4(active_cnt)) ||
        (union_cnt && !aligned4(union_cnt)) || (debug_z && !aligned4(debug_z)))
        return SFFN_ERR_INVALID_ARG;
    if (n_tokens == 0) return SFFN_OK;
    const bool batched = n_tokens > kDecodeMaxTokens;
    if (batched) {
        // The union path runs bf16 MFMA with a full gate.
        if (s.dtype != SFFN_BF16 || mode == SFFN_LOPA) return SFFN_ERR_UNSUPPORTED;
    }

    // ---- device set-up (first forward only) ----
    if (handle->n_cu == 0) {
        if (device_setup(*handle) != hipSuccess) return SFFN_ERR_HIP;
    }
    if (!batched && !decode_fits(*handle, n_tokens, mode)) return SFFN_ERR_UNSUPPORTED;

    FwdArgs a;
    a.x = x;
    a.n = n_tokens;
    a.w = *w;
    a.mode = mode;
    a.tau = tau;
    a.k = k;
    a.y = y;
    a.active_idx = active_idx;
    a.active_cnt = active_cnt;
    a.union_cnt = union_cnt;
    a.debug_z = debug_z;
    a.stream = static_cast<hipStream_t>(stream);

    if (!handle->inited) {
        if (launch_init(*handle, a.stream) != hipSuccess) return SFFN_ERR_HIP;
        handle->inited = true;
    }
    hipError_t e = batched ? launch_batched(*handle, a) : launch_decode(*handle, a);
    if (e != hipSuccess) {
        handle->inited = false;  // counters may be stale: re-zero on the next forward
        return e == hipErrorNotSupported ? SFFN_ERR_UNSUPPORTED : SFFN_ERR_HIP;
    }
    return SFFN_OK;
}

}  // extern "C"
