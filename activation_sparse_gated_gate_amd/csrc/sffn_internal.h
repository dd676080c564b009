// Internal declarations shared by the C ABI (abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "../../include/sffn.h"

namespace sffn {

constexpr int kMaxDffConst = 262144;
constexpr int kMaxDff = kMaxDffConst;

// Token grouping of large batches (groups.hip): at most this many groups,
// this many assignment rounds, and at least this many tokens per group.
constexpr int kMaxTokenGroups = 8;
constexpr int kTokenGroupIters = 4;
constexpr int kTokenGroupMinTokens = 64;

// Token counts up to this use the GEMV kernels (each weight row read once for
// all tokens); larger batches use the MFMA union path.
constexpr int kDecodeMaxTokens = 8;

// Control block (int32 slots) at the start of the workspace, zeroed by the
// first forward on a handle; reserved for counters of the batched path.
constexpr int kCtrlInts = 1024;
constexpr int kCtrlUnionSize = 0;    // batched path: size of the union list
constexpr int kCtrlError = 1;        // sticky error word (bits kErr*), workspace byte offset 4
constexpr int kCtrlEpoch = 2;        // decode forward counter (epoch of the slots), advanced by the gate kernel
constexpr int kCtrlUnionTrue = 3;    // batched path over every channel: the union bitmap's size
constexpr int kErrDownWait = 1;      // a down-projection sum gave up waiting for a group's slot

// Polls after which a waiting workgroup gives up (sffn_set_spin_limit).
constexpr int kSpinMaxDefault = 1 << 18;

// K splits of a batched GEMM (partial slices): up to 16 below 65 tokens, 8 up
// to 511 tokens, none from 512.
constexpr int kSplitMax = 16;
inline int splits_max(int T) { return T <= 64 ? 16 : T < 512 ? 8 : 1; }

constexpr int kDownGroupsMax = 64;   // channel groups of the split down projection
constexpr int kDownSliceCols = 128;  // output columns per down-projection workgroup
// Decode Top-K boundary slots: 8 sets x kDecodeMaxTokens tokens x {boundary bin, key, cutoff, prefetch estimate}.
constexpr int kTopkSlots = 8 * 8 * 4;
// compute units the batched partial buffer is sized for (the up GEMM's split
// rest needs one round of 256 x 256 tiles; on more CUs it runs in one launch)
constexpr int kUpRestCUs = 256;
constexpr int kDownRangeMax = 8192;  // channels of one down-projection group (32 per thread)
static_assert(kMaxDffConst <= kDownGroupsMax * kDownRangeMax, "the widest layer fits the groups");
// Channel groups of the decode down projection for d_ff = F: 16, so that the
// summing workgroup polls the 15 others' slots in one batch (32 at once made
// the wait twice as long), more for very wide layers so that a group has at
// most kDownRangeMax channels, at most F.
inline int down_groups(int F)
{
    const int G = (F + kDownRangeMax - 1) / kDownRangeMax;
    return F < 16 ? F : G > 16 ? G : 16;
}


struct Layout {
    int words;        // ceil(d_ff / 32)
    int ntp;          // padded decode token count (8)
    size_t ctrl;      // int32 [kCtrlInts]
    size_t act;       // uint8 [max(ntp, max_tokens)][d_ff]  per-token active flags (0/1)
    size_t gsel;      // decode: fp32 [ntp][d_ff] gate values; batched: bf16 [T][d_ff]
    size_t uidx;      // int32 [d_ff] ascending union list
    size_t hbuf;      // decode: fp32 [d_ff][ntp] gated up values; batched: bf16 [T][d_ff]
    size_t any;       // decode: uint8 [d_ff] union of the tokens' active flags
    size_t part;      // decode: 64-bit slots [down_groups - 1][ntp][d_model] down-projection group sums
    size_t part_slots;
    size_t tslot;     // decode Top-K: 64-bit slots [8 sets][8 tokens][4] of the per-token boundaries
    size_t tvec;      // fp32 [ntp][rank] LoPA x.A
    size_t keys;      // batched Top-K: fp32 [T][d_ff] SiLU keys
    size_t ubits;     // batched: uint32 [words] union bitmap
    size_t bpart;     // batched split-K partials: fp32 [bpart_rows][max(d_ff, d_model)]
    int bpart_rows;   // splits x tokens that fit in bpart
    size_t bpart_elems;  // fp32 elements of bpart
    // batched token grouping (groups.hip)
    size_t gbits;     // uint32 [T][words] per-token channel masks
    size_t gcnt;      // int32 [kMaxTokenGroups][d_ff] per-group channel counts
    size_t gstat;     // int32 [kMaxTokenGroups] sizes, then int64 [kMaxTokenGroups] sums of squares
    size_t grp;       // int32 [T] group of each token
    size_t tmap;      // int32 [T] tokens in group order
    size_t xp;        // bf16 [T][d_model] x in group order
    size_t gub;       // uint32 [kMaxTokenGroups][words] union bitmap of each group
    size_t guidx;     // int32 [kMaxTokenGroups][d_ff] union list of each group
    size_t gcount;    // int32 [kMaxTokenGroups] union size of each group
    size_t total;
};

bool shape_ok(const sffn_shape &s);
Layout make_layout(const sffn_shape &s);

struct FwdArgs {
    const void *x;
    int n;
    sffn_weights w;
    int mode;
    float tau;
    int k;
    float *y;
    int32_t *active_idx;
    int32_t *active_cnt;
    int32_t *union_cnt;
    float *debug_z;
    hipStream_t stream;
    float *usave = nullptr;  // training forward: fp32 [n][d_ff] up values of the union's channels
};

// Token grouping of a batch (groups.hip): groups by k-means on the tokens'
// channel masks (from G != 0), then each group's union bitmap (gub), the
// tokens in group order (tmap) and x in that order (xp); the batch's union
// size into *ncount and its bitmap cleared. Synchronises the stream once to
// return the group sizes in n_host[ng].
struct GroupArgs {
    int T, F, d, ng;
    const uint16_t *G;    // [T][F] bf16 gate values, 0 where off
    const uint16_t *x;    // [T][d]
    uint32_t *ubits;      // the batch's union bitmap
    int *ncount;
    uint32_t *Mb;
    int *cnt, *nsz;
    long long *Q;
    int *grp, *tmap;
    uint16_t *xp;
    uint32_t *gub;
    hipStream_t stream;
};
hipError_t launch_token_groups(const GroupArgs &a, int *n_host);

// Training workspace (sffn_train_workspace_bytes): buffers of the training
// forward's save step and of the backward, for up to T = max_tokens tokens.
struct TrainLayout {
    int tp_max;       // max_tokens rounded up to 8
    size_t zu;        // backward: float2 [T][d_ff] stored (z, u), z = NaN where off;
                      // forward: fp32 [T][d_ff] z, then fp32 [T][d_ff] u
    size_t du, dz;    // bf16 [T][FP] dU, dZ (token major; FP = d_ff rounded up to 8)
    size_t dut, dzt, ht;  // bf16 [FP][tp] dU, dZ, g(z) u transposed (union position major)
    size_t xt, dyt;   // bf16 [d_model][tp] x and dy transposed
    size_t ubits;     // uint32 [words] union of the stored sets
    size_t uidx;      // int32 [d_ff] ascending union list
    size_t ctrl;      // int32 [64]: union size
    size_t part;      // fp32 [part_rows][max(d_ff, d_model)] split-K partials
    int part_rows;
    size_t total;
};
TrainLayout make_train_layout(const sffn_shape &s);

// Stored activations of a training forward (per token, ascending channels).
struct Saved {
    int cap;
    int32_t *cnt, *idx;
    float *z, *u;
};

struct BwdArgs {
    const void *x, *dy;
    int n;
    sffn_weights w;
    int mode;
    float tau;
    Saved sv;
    float *dx, *dwg, *dwu, *dwd;
    char *tws;  // training workspace
    hipStream_t stream;
};

}  // namespace sffn

struct sffn_ctx {
    sffn_shape shape;
    char *ws;
    size_t ws_bytes;
    sffn::Layout L;
    bool inited;        // control block zeroed on the device
    int n_cu;           // compute units, read on the first forward
    int spin_max;       // polls before a waiting workgroup gives up
    int token_groups;   // batched forwards of enough tokens: this many token groups (<= 1: one union)
    void *ev_start;     // optional hipEvent_t pair around the dominant kernel
    void *ev_stop;
};

namespace sffn {
// Host checks of a forward's arguments against a shape (nothing is enqueued):
// SFFN_OK or the status to return.
sffn_status forward_checks(const sffn_shape &s, const void *x, int n_tokens, const sffn_weights *w, int mode,
                           float tau, int k, const float *y, const int32_t *active_idx, const int32_t *active_cnt,
                           const int32_t *union_cnt, const float *debug_z);
FwdArgs make_fwd(const void *x, int n_tokens, const sffn_weights *w, int mode, float tau, int k, float *y,
                 int32_t *active_idx, int32_t *active_cnt, int32_t *union_cnt, float *debug_z, void *stream);
// Enqueue a checked forward of n_tokens >= 1 on a set-up handle.
sffn_status forward_enqueue(sffn_ctx &c, const FwdArgs &a);
hipError_t device_setup(sffn_ctx &c);
hipError_t launch_init(sffn_ctx &c, hipStream_t s);
hipError_t launch_decode(sffn_ctx &c, const FwdArgs &a);
hipError_t launch_batched(sffn_ctx &c, const FwdArgs &a);
// Training (batched.hip): the forward on the union path plus the stored
// activations, and the backward over them.
hipError_t launch_forward_train(sffn_ctx &c, FwdArgs a, const Saved &sv, char *tws);
hipError_t launch_backward(sffn_ctx &c, const BwdArgs &a);
// Training helper kernels (train.hip).
// The saved rows of each token from the forward's dense z [T][F], up values
// [T][F] and flags: the channels the mode keeps, ascending, the first cap of
// them stored; cnt[t] = how many there are.
hipError_t launch_save(const float *zd, const float *ud, const uint8_t *act, int T, int F, int mode, float tau,
                       const Saved &sv, hipStream_t st);
// Backward set-up: (z, u) of the stored channels into ZU [T][F] (NaN z
// elsewhere), the union bitmap and ascending list of the stored channels
// (uidx, *ucount), zeroed token padding [T, tp) of the transposed buffers'
// rows, and x, dy transposed into xt, dyt [d][tp] (zero past T).
hipError_t launch_bwd_setup(const Saved &sv, int T, int F, int d, int tp, float2 *ZU, uint32_t *ubits,
                            int32_t *uidx, int *ucount, uint16_t *dut, uint16_t *dzt, uint16_t *ht,
                            const uint16_t *x, const uint16_t *dy, uint16_t *xt, uint16_t *dyt, hipStream_t st);
// Top-p: the same per-token pair, found by cumulative softmax mass p
// (decode), and the batched select + flags.
hipError_t launch_topp_select_flags(const float *keys, int T, int F, float p, uint8_t *act, uint16_t *G,
                                   uint32_t *ubits, hipStream_t st);
// The union bitmap from the flags act [T][F] (replaces whatever it holds).
hipError_t launch_union_flags(const uint8_t *act, int T, int F, uint32_t *ubits, hipStream_t st);
// A small batch whose up GEMM ran over every channel in the gate's launch:
// its split-K partials [S][T][F] (the gate's split count). A select kernel
// given them also writes the product rows H[t][i] = bf16(G[t][i] u[t][i]),
// u the partials summed in split order, zeros in the pad columns up to hld,
// u into usave when set, and the identity union list and its size (every
// channel) for the down GEMM. part null: none of this.
constexpr int kSelectUpMaxSplits = 4;
struct UpHalf {
    const float *part;
    uint16_t *H;
    int hld;
    float *usave;
    int32_t *uidx;
    int *ucount;
};

// Batched 2:8: act[t][i], bf16 gate values G[t][i] and the union bitmap from
// the keys (or from the gate GEMM's S split-K partials when part is set), keeping
// the top 2 of every aligned group of 8 channels.
hipError_t launch_nm_flags(const float *keys, int T, int F, uint8_t *act, uint16_t *G, uint32_t *ubits,
                           hipStream_t st, const float *part = nullptr, int S = 0, float *debug_z = nullptr,
                           const UpHalf &up = UpHalf{});
// Batched: the per-token select, then act[t][i], the bf16 gate values
// G[t][i] and the union bitmap words from it.
hipError_t launch_topk_select_flags(const float *keys, int T, int F, int K, uint8_t *act, uint16_t *G,
                                   uint32_t *ubits, hipStream_t st);
// Small batches whose gate GEMM split K: the per-token Top-K (K) or top-p
// (p) select straight from the S split-K partials [S][T][F] (summed in split
// order, then SiLU; the sums into debug_z when it is set), then its flags
// as launch_topk_select_flags; sum_select_fits says whether F and S allow it.
// The up half is taken with at most kSelectUpMaxSplits splits.
bool sum_select_fits(int F, int S);
hipError_t launch_sum_select_flags(const float *part, int S, int T, int F, int mode, int K, float p, float *debug_z,
                                   uint8_t *act, uint16_t *G, uint32_t *ubits, hipStream_t st,
                                   const UpHalf &up = UpHalf{});
// Decode gate kernel (gate.hip): gate GEMV + activation + select (+ the up
// rows of the selected channels, or of every channel in the dense modes).
struct GateArgs {
    int dtype;            // sffn_dtype of weights and x
    bool lopa;            // gate rows are B (length L) dotted with t = x.A (fp32, in xg)
    int nt;               // padded token count: 1, 2, 4 or 8
    int kind;             // GateKind (rowdot.h)
    int lpr;              // lanes per row group: 16, 32 or 64
    const void *xg;       // gate input [n][L]: x, or t = x.A for LoPA
    int n, L;
    const void *xu;       // up input x [n][d]
    int d;
    const void *wg, *wu;  // gate rows [F][L] (B for LoPA), up rows [F][d]
    int F, mode;
    float tau;
    float *gsel;          // [8][F] gate values / Top-K keys
    uint8_t *act;         // [8][F] selected flags (threshold)
    uint8_t *any;         // [F] union of the selected flags over the tokens
    float *hbuf;          // [F][8] h values of selected channels
    float *debug_z;
    hipStream_t stream;
    void *ev_start, *ev_stop;  // optional: this kernel's own begin / end timestamps
    int *ctrl;            // control block: the gate kernel advances the decode epoch
};
hipError_t launch_gate(const GateArgs &g);
}  // namespace sffn
