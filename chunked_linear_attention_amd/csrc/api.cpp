// C ABI of libttt_mi355x.so: argument validation, workspace queries, dispatch.
// Every check runs on the host before anything is enqueued; on any error
// nothing is written.
#include "../../include/ttt.h"
#include "ttt_internal.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_enums(int dtype, int loss, int order)
{
    return (dtype == TTT_F32 || dtype == TTT_BF16) && (loss == TTT_LOSS_DOT || loss == TTT_LOSS_MSE) &&
           (order == TTT_CAUSAL || order == TTT_NONCAUSAL);
}

// Shape checks common to both ops.  Returns TTT_OK or an error code.
ttt_status check_dims(int B, int H, int Tq, int Tkv, int d, int chunk, int order)
{
    if (B < 1 || H < 1 || d < 1 || chunk < 1 || Tq < 0 || Tkv < 0) return TTT_EINVAL;
    if (order == TTT_CAUSAL && Tq != Tkv) return TTT_EINVAL;
    // element counts must fit the kernels' 32-bit token indices
    if ((long long)Tq > (1LL << 30) || (long long)Tkv > (1LL << 30)) return TTT_EUNSUPPORTED;
    if ((long long)B * H > (1LL << 24)) return TTT_EUNSUPPORTED;
    return TTT_OK;
}

bool linear_supported(int d, int chunk) { return (d == 64 || d == 128) && chunk % 16 == 0; }

// The LaCT kernels tile d and hidden by 128 (GEMM tiles) and never let a
// 128-token tile straddle two chunks.
bool lact_supported(int dtype, int d, int hid, int chunk, int Tkv)
{
    if (dtype != TTT_BF16) return false;
    if (d % 128 != 0 || hid % 128 != 0 || d > 1024 || hid > 1024) return false;
    if (!(chunk % 128 == 0 || chunk >= Tkv)) return false;
    return true;
}

// [a, a + na) and [b, b + nb) share a byte
bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace

extern "C" {

const char *ttt_status_string(int status)
{
    switch (status) {
    case TTT_OK: return "ok";
    case TTT_EINVAL: return "invalid argument";
    case TTT_EUNSUPPORTED: return "unsupported shape or dtype";
    case TTT_EWORKSPACE: return "workspace too small";
    case TTT_EHIP: return "HIP error";
    default: return "unknown status";
    }
}

int ttt_abi_version(void) { return 3; }

size_t ttt_linear_workspace_bytes_seg(int B, int H, int Tq, int Tkv, int d, int chunk, int loss,
                                      int order, int dtype, int seg_tokens)
{
    if (!valid_enums(dtype, loss, order) || seg_tokens < 0) return 0;
    if (check_dims(B, H, Tq, Tkv, d, chunk, order) != TTT_OK) return 0;
    if (!linear_supported(d, chunk)) return 0;
    tttk::LinearShape s{B * H, Tq, Tkv, d, chunk, loss, order, dtype == TTT_BF16 ? 1 : 0, seg_tokens};
    return tttk::linear_plan(s).bytes;
}

size_t ttt_linear_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int chunk, int loss,
                                  int order, int dtype)
{
    return ttt_linear_workspace_bytes_seg(B, H, Tq, Tkv, d, chunk, loss, order, dtype, 0);
}

ttt_status ttt_linear_fwd_seg(const void *q, const void *k, const void *v, int dtype,
                              const float *eta, const float *w_init, void *out, float *w_final,
                              int B, int H, int Tq, int Tkv, int d, int chunk, int loss, int order,
                              int seg_tokens, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!valid_enums(dtype, loss, order) || seg_tokens < 0) return TTT_EINVAL;
    ttt_status st = check_dims(B, H, Tq, Tkv, d, chunk, order);
    if (st != TTT_OK) return st;
    if (!w_init || !w_final || !aligned16(w_init) || !aligned16(w_final)) return TTT_EINVAL;
    if (Tq > 0 && (!q || !out || !aligned16(q) || !aligned16(out))) return TTT_EINVAL;
    if (Tkv > 0 && (!k || !v || !eta || !aligned16(k) || !aligned16(v) || !aligned16(eta)))
        return TTT_EINVAL;
    if (!linear_supported(d, chunk)) return TTT_EUNSUPPORTED;
    tttk::LinearShape s{B * H, Tq, Tkv, d, chunk, loss, order, dtype == TTT_BF16 ? 1 : 0, seg_tokens};
    tttk::LinearPlan pl = tttk::linear_plan(s);
    if (pl.bytes > 0 && (!workspace || !aligned16(workspace))) return TTT_EINVAL;
    if (workspace_bytes < pl.bytes) return TTT_EWORKSPACE;
    hipError_t e = tttk::linear_launch(s, pl, q, k, v, eta, w_init, out, w_final, workspace,
                                       (hipStream_t)stream);
    return e == hipSuccess ? TTT_OK : TTT_EHIP;
}

ttt_status ttt_linear_fwd(const void *q, const void *k, const void *v, int dtype, const float *eta,
                          const float *w_init, void *out, float *w_final, int B, int H, int Tq,
                          int Tkv, int d, int chunk, int loss, int order, void *workspace,
                          size_t workspace_bytes, void *stream)
{
    return ttt_linear_fwd_seg(q, k, v, dtype, eta, w_init, out, w_final, B, H, Tq, Tkv, d, chunk,
                              loss, order, 0, workspace, workspace_bytes, stream);
}

size_t lact_swiglu_rule_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int hidden,
                                        int chunk, int loss, int order, int dtype, int rule)
{
    if (!valid_enums(dtype, loss, order) || rule < TTT_RULE_GD || rule > TTT_RULE_MUON) return 0;
    if (check_dims(B, H, Tq, Tkv, d, chunk, order) != TTT_OK || hidden < 1) return 0;
    if (!lact_supported(dtype, d, hidden, chunk, Tkv)) return 0;
    tttk::LactShape s{B * H, Tq, Tkv, d, hidden, chunk, loss, order, 1};
    s.rule = rule;
    return tttk::lact_plan(s).bytes;
}

size_t lact_swiglu_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int hidden, int chunk,
                                   int loss, int order, int dtype)
{
    return lact_swiglu_rule_workspace_bytes(B, H, Tq, Tkv, d, hidden, chunk, loss, order, dtype,
                                            TTT_RULE_GD);
}

ttt_status lact_swiglu_fwd_rule(const void *q, const void *k, const void *v, int dtype,
                                const float *eta, const float *w1_init, const float *w2_init,
                                const float *w3_init, void *out, float *w1_final, float *w2_final,
                                float *w3_final, int B, int H, int Tq, int Tkv, int d, int hidden,
                                int chunk, int loss, int order, int rownorm, int rule, float beta,
                                int ns_steps, float muon_lr, float *m1, float *m2, float *m3,
                                void *workspace, size_t workspace_bytes, void *stream,
                                void *aux_stream)
{
    if (!valid_enums(dtype, loss, order)) return TTT_EINVAL;
    ttt_status st = check_dims(B, H, Tq, Tkv, d, chunk, order);
    if (st != TTT_OK) return st;
    if (hidden < 1 || (rownorm != 0 && rownorm != 1)) return TTT_EINVAL;
    const void *ws_ptrs[6] = {w1_init, w2_init, w3_init, w1_final, w2_final, w3_final};
    for (const void *p : ws_ptrs)
        if (!p || !aligned16(p)) return TTT_EINVAL;
    if (Tq > 0 && (!q || !out || !aligned16(q) || !aligned16(out))) return TTT_EINVAL;
    if (Tkv > 0 && (!k || !v || !eta || !aligned16(k) || !aligned16(v) || !aligned16(eta)))
        return TTT_EINVAL;
    // update rule: the momentum coefficient lies in [0, 1]; Muon takes 1..16
    // Newton-Schulz steps and a finite step size >= 0
    if (rule < TTT_RULE_GD || rule > TTT_RULE_MUON) return TTT_EINVAL;
    if (rule != TTT_RULE_GD && !(beta >= 0.f && beta <= 1.f)) return TTT_EINVAL;
    if (rule == TTT_RULE_MUON && (ns_steps < 1 || ns_steps > 16 || !(muon_lr >= 0.f) ||
                                  muon_lr > 3.0e38f))
        return TTT_EINVAL;
    const bool use_m = rule == TTT_RULE_MOMENTUM || (rule == TTT_RULE_MUON && beta != 0.f);
    if (use_m) {
        const float *ms[3] = {m1, m2, m3};
        for (const float *p : ms)
            if (!p || !aligned16(p)) return TTT_EINVAL;
    }
    if (!lact_supported(dtype, d, hidden, chunk, Tkv)) return TTT_EUNSUPPORTED;
    tttk::LactShape s{B * H, Tq, Tkv, d, hidden, chunk, loss, order, rownorm};
    s.rule = rule;
    s.beta = rule == TTT_RULE_GD ? 0.f : beta;
    s.ns_steps = rule == TTT_RULE_MUON ? ns_steps : 0;
    s.lr = rule == TTT_RULE_MUON ? muon_lr : 0.f;
    tttk::LactPlan pl = tttk::lact_plan(s);
    if (pl.bytes > 0 && (!workspace || !aligned16(workspace))) return TTT_EINVAL;
    if (workspace_bytes < pl.bytes) return TTT_EWORKSPACE;
    hipError_t e = tttk::lact_launch(s, pl, q, k, v, eta, w1_init, w2_init, w3_init, out, w1_final,
                                     w2_final, w3_final, workspace, (hipStream_t)stream,
                                     (hipStream_t)aux_stream, use_m ? m1 : nullptr,
                                     use_m ? m2 : nullptr, use_m ? m3 : nullptr);
    return e == hipSuccess ? TTT_OK : TTT_EHIP;
}

size_t lact_swiglu_bwd_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int hidden, int chunk,
                                       int loss, int order, int dtype)
{
    if (!valid_enums(dtype, loss, order)) return 0;
    if (check_dims(B, H, Tq, Tkv, d, chunk, order) != TTT_OK || hidden < 1 || Tkv < 1) return 0;
    if (!lact_supported(dtype, d, hidden, chunk, Tkv) || loss != TTT_LOSS_DOT) return 0;
    tttk::LactShape s{B * H, Tq, Tkv, d, hidden, chunk, loss, order, 1};
    return tttk::lact_bwd_plan(s).bytes;
}

ttt_status lact_swiglu_bwd(const void *q, const void *k, const void *v, int dtype, const float *eta,
                           const float *w1_init, const float *w2_init, const float *w3_init,
                           const void *d_out, const float *d_w1_final, const float *d_w2_final,
                           const float *d_w3_final, void *d_q, void *d_k, void *d_v, float *d_eta,
                           float *d_w1_init, float *d_w2_init, float *d_w3_init, int B, int H,
                           int Tq, int Tkv, int d, int hidden, int chunk, int loss, int order,
                           int rownorm, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!valid_enums(dtype, loss, order)) return TTT_EINVAL;
    ttt_status st = check_dims(B, H, Tq, Tkv, d, chunk, order);
    if (st != TTT_OK) return st;
    if (hidden < 1 || Tkv < 1 || (rownorm != 0 && rownorm != 1)) return TTT_EINVAL;
    const void *need[10] = {k, v, eta, w1_init, w2_init, w3_init, d_k, d_v, d_eta, d_w1_init};
    for (const void *p : need)
        if (!p || !aligned16(p)) return TTT_EINVAL;
    if (!d_w2_init || !d_w3_init || !aligned16(d_w2_init) || !aligned16(d_w3_init)) return TTT_EINVAL;
    if (Tq > 0 && (!q || !d_out || !d_q || !aligned16(q) || !aligned16(d_out) || !aligned16(d_q)))
        return TTT_EINVAL;
    // the upstream weight gradients come as all three or none
    const int ndw = (d_w1_final != nullptr) + (d_w2_final != nullptr) + (d_w3_final != nullptr);
    if (ndw != 0 && ndw != 3) return TTT_EINVAL;
    if (ndw == 3 && (!aligned16(d_w1_final) || !aligned16(d_w2_final) || !aligned16(d_w3_final)))
        return TTT_EINVAL;
    if (!lact_supported(dtype, d, hidden, chunk, Tkv) || loss != TTT_LOSS_DOT) return TTT_EUNSUPPORTED;
    // outputs must not overlap the inputs or each other
    const size_t NH = (size_t)B * H, n13 = (size_t)hidden * d;
    const size_t tk = NH * Tkv * d * 2, tq = NH * (size_t)Tq * d * 2, te = NH * Tkv * 4, tw = NH * n13 * 4;
    const void *outs[7] = {d_q, d_k, d_v, d_eta, d_w1_init, d_w2_init, d_w3_init};
    const size_t osz[7] = {tq, tk, tk, te, tw, tw, tw};
    const void *ins[11] = {q, k, v, eta, w1_init, w2_init, w3_init, d_out, d_w1_final, d_w2_final, d_w3_final};
    const size_t isz[11] = {tq, tk, tk, te, tw, tw, tw, tq, tw, tw, tw};
    for (int a = 0; a < 7; ++a) {
        if (!outs[a] || osz[a] == 0) continue;
        for (int b = 0; b < 11; ++b)
            if (ins[b] && isz[b] && overlaps(outs[a], osz[a], ins[b], isz[b])) return TTT_EINVAL;
        for (int b = a + 1; b < 7; ++b)
            if (outs[b] && osz[b] && overlaps(outs[a], osz[a], outs[b], osz[b])) return TTT_EINVAL;
    }
    tttk::LactShape s{B * H, Tq, Tkv, d, hidden, chunk, loss, order, rownorm};
    tttk::LactBwdPlan pl = tttk::lact_bwd_plan(s);
    if (!workspace || !aligned16(workspace)) return TTT_EINVAL;
    if (workspace_bytes < pl.bytes) return TTT_EWORKSPACE;
    hipError_t e = tttk::lact_bwd_launch(s, pl, q, k, v, eta, w1_init, w2_init, w3_init, d_out,
                                         d_w1_final, d_w2_final, d_w3_final, d_q, d_k, d_v, d_eta,
                                         d_w1_init, d_w2_init, d_w3_init, workspace,
                                         (hipStream_t)stream);
    return e == hipSuccess ? TTT_OK : TTT_EHIP;
}

ttt_status lact_swiglu_fwd(const void *q, const void *k, const void *v, int dtype,
                           const float *eta, const float *w1_init, const float *w2_init,
                           const float *w3_init, void *out, float *w1_final, float *w2_final,
                           float *w3_final, int B, int H, int Tq, int Tkv, int d, int hidden,
                           int chunk, int loss, int order, int rownorm, void *workspace,
                           size_t workspace_bytes, void *stream, void *aux_stream)
{
    return lact_swiglu_fwd_rule(q, k, v, dtype, eta, w1_init, w2_init, w3_init, out, w1_final,
                                w2_final, w3_final, B, H, Tq, Tkv, d, hidden, chunk, loss, order,
                                rownorm, TTT_RULE_GD, 0.f, 0, 0.f, nullptr, nullptr, nullptr,
                                workspace, workspace_bytes, stream, aux_stream);
}

ttt_status ttt_linear_decode(const void *q, const void *k, const void *v, int dtype,
                             const float *eta, float *w, float *w_anchor, int anchor_update,
                             void *out, int B, int H, int d, int loss, void *stream)
{
    if (!valid_enums(dtype, loss, TTT_CAUSAL)) return TTT_EINVAL;
    if (B < 1 || H < 1 || d < 1 || (anchor_update != 0 && anchor_update != 1)) return TTT_EINVAL;
    if ((long long)B * H > (1LL << 24)) return TTT_EUNSUPPORTED;
    const void *req[6] = {q, k, v, eta, w, out};
    for (const void *p : req)
        if (!p || !aligned16(p)) return TTT_EINVAL;
    if (anchor_update && !w_anchor) return TTT_EINVAL;
    if (d != 64 && d != 128) return TTT_EUNSUPPORTED;
    const size_t sbytes = (size_t)B * H * d * d * sizeof(float);
    if (w_anchor && (!aligned16(w_anchor) || overlaps(w, sbytes, w_anchor, sbytes)))
        return TTT_EINVAL;
    hipError_t e = tttk::linear_decode_launch(B * H, d, dtype == TTT_BF16 ? 1 : 0, loss, q, k, v,
                                              eta, w, w_anchor, anchor_update, out,
                                              (hipStream_t)stream);
    return e == hipSuccess ? TTT_OK : TTT_EHIP;
}

size_t lact_swiglu_decode_workspace_bytes(int B, int H, int d, int hidden, int dtype)
{
    if ((dtype != TTT_F32 && dtype != TTT_BF16) || B < 1 || H < 1 || d < 1 || hidden < 1) return 0;
    if ((long long)B * H > (1LL << 24) || d % 64 || hidden % 64 || d > 1024 || hidden > 1024)
        return 0;
    return tttk::lact_decode_workspace(B * H, hidden);
}

ttt_status lact_swiglu_decode(const void *q, int dtype, const float *w1, const float *w2,
                              const float *w3, void *out, int B, int H, int d, int hidden,
                              void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != TTT_F32 && dtype != TTT_BF16) return TTT_EINVAL;
    if (B < 1 || H < 1 || d < 1 || hidden < 1) return TTT_EINVAL;
    const void *req[6] = {q, w1, w2, w3, out, workspace};
    for (const void *p : req)
        if (!p || !aligned16(p)) return TTT_EINVAL;
    if ((long long)B * H > (1LL << 24)) return TTT_EUNSUPPORTED;
    if (d % 64 || hidden % 64 || d > 1024 || hidden > 1024) return TTT_EUNSUPPORTED;
    if (workspace_bytes < tttk::lact_decode_workspace(B * H, hidden)) return TTT_EWORKSPACE;
    hipError_t e = tttk::lact_decode_launch(B * H, d, hidden, dtype == TTT_BF16 ? 1 : 0, q, w1, w2,
                                            w3, out, workspace, (hipStream_t)stream);
    return e == hipSuccess ? TTT_OK : TTT_EHIP;
}

ttt_status window_attention_fwd(const void *q, const void *k, const void *v, int dtype, void *out,
                                int B, int H, int T, int d, int window, float scale,
                                int accumulate, void *stream)
{
    if (dtype != TTT_F32 && dtype != TTT_BF16) return TTT_EINVAL;
    if (B < 1 || H < 1 || T < 0 || d < 1 || window < 1) return TTT_EINVAL;
    if (accumulate != 0 && accumulate != 1) return TTT_EINVAL;
    if (!(scale > 0.f) || scale > 3.0e38f) return TTT_EINVAL;
    if (T > 0) {
        const void *req[4] = {q, k, v, out};
        for (const void *p : req)
            if (!p || !aligned16(p)) return TTT_EINVAL;
    }
    if ((long long)B * H > (1LL << 24) || (long long)T > (1LL << 30)) return TTT_EUNSUPPORTED;
    if (dtype != TTT_BF16 || (d != 64 && d != 128 && d != 256)) return TTT_EUNSUPPORTED;
    if (T == 0) return TTT_OK;
    if ((long long)B * H * ((T + 127) / 128) > 0x7fffffffLL) return TTT_EUNSUPPORTED;
    hipError_t e = tttk::window_attn_launch(B * H, T, d, window, scale, accumulate, q, k, v, out,
                                            (hipStream_t)stream);
    return e == hipSuccess ? TTT_OK : TTT_EHIP;
}

size_t ttt_linear_bwd_workspace_bytes(int B, int H, int Tq, int Tkv, int d, int chunk, int loss,
                                      int order, int dtype)
{
    if (!valid_enums(dtype, loss, order) || B < 1 || H < 1 || Tq < 0 || Tkv < 1) return 0;
    if (order == TTT_CAUSAL && Tq != Tkv) return 0;
    if ((long long)B * H > (1LL << 24) || (long long)Tq > (1LL << 30) || (long long)Tkv > (1LL << 30))
        return 0;
    if (!linear_supported(d, chunk)) return 0;
    return tttk::linear_bwd_workspace(B * H, Tkv, d, chunk);
}

ttt_status ttt_linear_bwd(const void *q, const void *k, const void *v, int dtype, const float *eta,
                          const float *w_init, const void *d_out, const float *d_w_final,
                          void *d_q, void *d_k, void *d_v, float *d_eta, float *d_w_init, int B,
                          int H, int Tq, int Tkv, int d, int chunk, int loss, int order,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    if (!valid_enums(dtype, loss, order)) return TTT_EINVAL;
    if (B < 1 || H < 1 || Tq < 0 || Tkv < 1 || d < 1 || chunk < 1) return TTT_EINVAL;
    if (order == TTT_CAUSAL && Tq != Tkv) return TTT_EINVAL;
    const void *req[8] = {k, v, eta, w_init, d_k, d_v, d_eta, d_w_init};
    for (const void *p : req)
        if (!p || !aligned16(p)) return TTT_EINVAL;
    if (Tq > 0) {
        const void *qs[3] = {q, d_out, d_q};
        for (const void *p : qs)
            if (!p || !aligned16(p)) return TTT_EINVAL;
    }
    if (d_w_final && !aligned16(d_w_final)) return TTT_EINVAL;
    if ((long long)B * H > (1LL << 24) || (long long)Tq > (1LL << 30) || (long long)Tkv > (1LL << 30))
        return TTT_EUNSUPPORTED;
    if (!linear_supported(d, chunk)) return TTT_EUNSUPPORTED;
    const size_t need = tttk::linear_bwd_workspace(B * H, Tkv, d, chunk);
    if (!workspace || !aligned16(workspace)) return TTT_EINVAL;
    if (workspace_bytes < need) return TTT_EWORKSPACE;
    hipError_t e = tttk::linear_bwd_launch(B * H, Tq, Tkv, d, chunk, loss, order,
                                           dtype == TTT_BF16 ? 1 : 0, q, k, v, eta, w_init, d_out,
                                           d_w_final, d_q, d_k, d_v, d_eta, d_w_init, workspace,
                                           (hipStream_t)stream);
    return e == hipSuccess ? TTT_OK : TTT_EHIP;
}

}  // extern "C"
