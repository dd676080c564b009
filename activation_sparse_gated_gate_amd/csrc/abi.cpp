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
    L.part_slots = (size_t)(down_groups(s.d_ff) - 1) * ntp * d;
    L.part = take(L.part_slots * 8);
    L.tslot = take((size_t)kTopkSlots * 8);
    L.tvec = take(r ? ntp * r * 4 : 0);
    L.keys = take(rows * F * 4);  // also for a training forward of <= 8 tokens (union path)
    L.ubits = take((size_t)L.words * 4);
    // room for every split a forward of up to T tokens takes, at least 16
    // splits of 64 tokens (forwards smaller than the handle's maximum)
    const size_t prow = T < 512 ? (size_t)splits_max((int)T) * T : 0, pmin = 16 * (T < 64 ? T : 64);
    L.bpart_rows = batched ? (int)(prow > pmin ? prow : pmin) : 0;
    // and, from 512 tokens, one round of 256 x 256 tiles on kUpRestCUs CUs
    // (the split rest of the up GEMM)
    const size_t pel = (size_t)L.bpart_rows * (F > d ? F : d), pround = T >= 512 ? (size_t)kUpRestCUs * 65536 : 0;
    L.bpart_elems = pel > pround ? pel : pround;
    L.bpart = take(L.bpart_elems * 4);
    if (batched) {
        const size_t W = (size_t)L.words, NG = kMaxTokenGroups;
        L.gbits = take(T * W * 4);
        L.gcnt = take(NG * F * 4);
        L.gstat = take(NG * 4 + NG * 8);
        L.grp = take(T * 4);
        L.tmap = take(T * 4);
        L.xp = take(T * d * 2);
        L.gub = take(NG * W * 4);
        L.guidx = take(NG * F * 4);
        L.gcount = take(NG * 4);
    }
    L.total = off;
    return L;
}

TrainLayout make_train_layout(const sffn_shape &s)
{
    TrainLayout L{};
    const size_t F = (size_t)s.d_ff, d = (size_t)s.d_model, T = (size_t)s.max_tokens;
    const size_t FP = (F + 7) / 8 * 8, TP = (T + 7) / 8 * 8;
    L.tp_max = (int)TP;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align256(off + bytes + 256);  // 256 bytes of slack after every buffer
        return at;
    };
    L.zu = take(T * FP * 8);
    L.du = take(T * FP * 2);
    L.dz = take(T * FP * 2);
    L.dut = take(FP * TP * 2);
    L.dzt = take(FP * TP * 2);
    L.ht = take(FP * TP * 2);
    L.xt = take(d * TP * 2);
    L.dyt = take(d * TP * 2);
    L.ubits = take((F + 31) / 32 * 4);
    L.uidx = take(F * 4);
    L.ctrl = take(64 * 4);
    const size_t prow = T < 512 ? (size_t)splits_max((int)T) * T : 0, pmin = 16 * (T < 64 ? T : 64);
    L.part_rows = (int)(prow > pmin ? prow : pmin);
    L.part = take((size_t)L.part_rows * (F > d ? F : d) * 4);
    L.total = off;
    return L;
}

// Most channels a mode can keep per token: the Top-K size, the 2:8 count,
// or d_ff (threshold, top-p and the dense modes).
static int max_kept(int mode, int F, int k)
{
    if (mode == SFFN_TOPK) return k;
    if (mode == SFFN_TOPK_2_8) return (F / 8) * 2 + (F % 8 < 2 ? F % 8 : 2);
    return F;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
static bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

sffn_status forward_checks(const sffn_shape &s, const void *x, int n_tokens, const sffn_weights *w, int mode,
                           float tau, int k, const float *y, const int32_t *active_idx, const int32_t *active_cnt,
                           const int32_t *union_cnt, const float *debug_z)
{
    if (!w) return SFFN_ERR_INVALID_ARG;
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
    if (n_tokens > kDecodeMaxTokens) {
        // The union path runs bf16 MFMA with a full gate.
        if (s.dtype != SFFN_BF16 || mode == SFFN_LOPA) return SFFN_ERR_UNSUPPORTED;
    }
    return SFFN_OK;
}

FwdArgs make_fwd(const void *x, int n_tokens, const sffn_weights *w, int mode, float tau, int k, float *y,
                 int32_t *active_idx, int32_t *active_cnt, int32_t *union_cnt, float *debug_z, void *stream)
{
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
    return a;
}

// The one-time clears of the control block and union bitmap, before the
// first forward on a handle. A forward captured into a graph enqueues them
// into the graph and leaves the handle uninitialised: they run only when the
// graph is replayed, so the next eager forward clears again.
static hipError_t ensure_init(sffn_ctx &c, hipStream_t st)
{
    if (c.inited) return hipSuccess;
    hipError_t e = launch_init(c, st);
    if (e != hipSuccess) return e;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(st, &cs)) != hipSuccess) return e;
    c.inited = cs == hipStreamCaptureStatusNone;
    return hipSuccess;
}

sffn_status forward_enqueue(sffn_ctx &c, const FwdArgs &a)
{
    // launches report errors through the thread's last-error slot: clear what
    // an earlier call of the caller's may have left there
    (void)hipGetLastError();
    if (ensure_init(c, a.stream) != hipSuccess) return SFFN_ERR_HIP;
    const hipError_t e = a.n > kDecodeMaxTokens ? launch_batched(c, a) : launch_decode(c, a);
    if (e != hipSuccess) {
        c.inited = false;  // counters may be stale: re-zero on the next forward
        return e == hipErrorNotSupported ? SFFN_ERR_UNSUPPORTED : SFFN_ERR_HIP;
    }
    return SFFN_OK;
}

}  // namespace sffn

using namespace sffn;

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
    c->spin_max = kSpinMaxDefault;
    c->token_groups = 1;
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

sffn_status sffn_set_token_groups(sffn_handle handle, int groups)
{
    if (!handle || groups < 1 || groups > kMaxTokenGroups) return SFFN_ERR_INVALID_ARG;
    handle->token_groups = groups;
    return SFFN_OK;
}

sffn_status sffn_set_spin_limit(sffn_handle handle, int polls)
{
    if (!handle) return SFFN_ERR_INVALID_ARG;
    handle->spin_max = polls < -1 ? -1 : polls;
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
    if (!handle) return SFFN_ERR_INVALID_ARG;
    const sffn_status v =
        forward_checks(handle->shape, x, n_tokens, w, mode, tau, k, y, active_idx, active_cnt, union_cnt, debug_z);
    if (v != SFFN_OK || n_tokens == 0) return v;

    // ---- device set-up (first forward only) ----
    if (handle->n_cu == 0) {
        if (device_setup(*handle) != hipSuccess) return SFFN_ERR_HIP;
    }
    return forward_enqueue(*handle, make_fwd(x, n_tokens, w, mode, tau, k, y, active_idx, active_cnt, union_cnt,
                                             debug_z, stream));
}

size_t sffn_train_workspace_bytes(const sffn_shape *shape)
{
    if (!shape || !shape_ok(*shape)) return 0;
    return make_train_layout(*shape).total;
}

// Checks shared by the training forward and the backward; SFFN_OK or the
// status to return.
static sffn_status train_checks(sffn_handle handle, int n_tokens, const sffn_weights *w, int mode, float tau, int k,
                                const sffn_saved *saved, void *train_ws, size_t train_ws_bytes)
{
    if (!handle || !w || !saved) return SFFN_ERR_INVALID_ARG;
    const sffn_shape &s = handle->shape;
    if (n_tokens < 0 || n_tokens > s.max_tokens) return SFFN_ERR_INVALID_ARG;
    if (mode < SFFN_THRESHOLD || mode > SFFN_TOPP) return SFFN_ERR_INVALID_ARG;
    if (mode == SFFN_LOPA || s.dtype != SFFN_BF16) return SFFN_ERR_UNSUPPORTED;
    if (!w->w_gate || !w->w_up || !w->w_down || !aligned16(w->w_gate) || !aligned16(w->w_up) ||
        !aligned16(w->w_down))
        return SFFN_ERR_INVALID_ARG;
    if (mode == SFFN_TOPK && (k < 1 || k > s.d_ff)) return SFFN_ERR_INVALID_ARG;
    if (mode != SFFN_TOPK && mode != SFFN_TOPK_2_8 && std::isnan(tau)) return SFFN_ERR_INVALID_ARG;
    if (mode == SFFN_TOPP && !(tau > 0.f && tau <= 1.f)) return SFFN_ERR_INVALID_ARG;
    if (saved->cap < 1 || saved->cap > s.d_ff) return SFFN_ERR_INVALID_ARG;
    if ((mode == SFFN_TOPK || mode == SFFN_TOPK_2_8 || mode == SFFN_DENSE_SILU) &&
        saved->cap < max_kept(mode, s.d_ff, k))
        return SFFN_ERR_INVALID_ARG;
    if (!saved->cnt || !saved->idx || !saved->z || !saved->u || !aligned4(saved->cnt) || !aligned4(saved->idx) ||
        !aligned4(saved->z) || !aligned4(saved->u))
        return SFFN_ERR_INVALID_ARG;
    if (!train_ws || ((uintptr_t)train_ws & 255u) != 0 || train_ws_bytes < make_train_layout(s).total)
        return SFFN_ERR_WORKSPACE;
    return SFFN_OK;
}

static Saved to_saved(const sffn_saved *v) { return Saved{v->cap, v->cnt, v->idx, v->z, v->u}; }

sffn_status sffn_forward_train(sffn_handle handle, const void *x, int n_tokens, const sffn_weights *w, int mode,
                               float tau, int k, float *y, const sffn_saved *saved, void *train_ws,
                               size_t train_ws_bytes, void *stream)
{
    const sffn_status v = train_checks(handle, n_tokens, w, mode, tau, k, saved, train_ws, train_ws_bytes);
    if (v != SFFN_OK) return v;
    if (!x || !y || !aligned16(x) || !aligned16(y)) return SFFN_ERR_INVALID_ARG;
    if (n_tokens == 0) return SFFN_OK;
    if (handle->n_cu == 0) {
        if (device_setup(*handle) != hipSuccess) return SFFN_ERR_HIP;
    }
    const FwdArgs a = make_fwd(x, n_tokens, w, mode, tau, k, y, nullptr, nullptr, nullptr, nullptr, stream);
    (void)hipGetLastError();  // as in forward_enqueue
    if (ensure_init(*handle, a.stream) != hipSuccess) return SFFN_ERR_HIP;
    const hipError_t e = launch_forward_train(*handle, a, to_saved(saved), static_cast<char *>(train_ws));
    if (e != hipSuccess) {
        handle->inited = false;
        return e == hipErrorNotSupported ? SFFN_ERR_UNSUPPORTED : SFFN_ERR_HIP;
    }
    return SFFN_OK;
}

sffn_status sffn_backward(sffn_handle handle, const void *x, const void *dy, int n_tokens, const sffn_weights *w,
                          int mode, float tau, int k, const sffn_saved *saved, float *dx, float *dw_gate,
                          float *dw_up, float *dw_down, void *train_ws, size_t train_ws_bytes, void *stream)
{
    const sffn_status v = train_checks(handle, n_tokens, w, mode, tau, k, saved, train_ws, train_ws_bytes);
    if (v != SFFN_OK) return v;
    if (!x || !dy || !dx || !dw_gate || !dw_up || !dw_down || !aligned16(x) || !aligned16(dy) || !aligned16(dx) ||
        !aligned16(dw_gate) || !aligned16(dw_up) || !aligned16(dw_down))
        return SFFN_ERR_INVALID_ARG;
    if (n_tokens == 0) return SFFN_OK;
    if (handle->n_cu == 0) {
        if (device_setup(*handle) != hipSuccess) return SFFN_ERR_HIP;
    }
    BwdArgs a;
    a.x = x;
    a.dy = dy;
    a.n = n_tokens;
    a.w = *w;
    a.mode = mode;
    a.tau = tau;
    a.sv = to_saved(saved);
    a.dx = dx;
    a.dwg = dw_gate;
    a.dwu = dw_up;
    a.dwd = dw_down;
    a.tws = static_cast<char *>(train_ws);
    a.stream = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();  // as in forward_enqueue
    return launch_backward(*handle, a) == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}

}  // extern "C"
