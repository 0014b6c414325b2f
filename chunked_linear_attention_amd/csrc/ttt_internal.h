// Host-side interfaces between the C ABI layer (api.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace tttk {

// ---- TTT-Linear ---------------------------------------------------------------
struct LinearShape {
    int NH;       // batch * heads
    int Tq, Tkv;  // query and key/value tokens per head
    int d;        // head dim (64 or 128)
    int chunk;    // chunk size (multiple of 16)
    int loss;     // 0 inner product, 1 MSE
    int order;    // 0 causal, 1 non-causal
    int bf16;     // 1 bf16 inputs/outputs, 0 fp32
    int seg_tokens = 0;  // segment length chosen by the caller (0: the plan's own choice)
};

struct LinearPlan {
    int seg_tokens;   // tokens per segment (multiple of chunk and of 16)
    int S;            // segments over the key/value sequence
    int Ssum;         // segments whose affine summary is needed
    int seg_q;        // tokens per query segment (non-causal apply)
    int Sq;           // query segments (non-causal apply)
    size_t offP, offB, offW, bytes;  // workspace layout (bytes)
};

LinearPlan linear_plan(const LinearShape &s);
hipError_t linear_launch(const LinearShape &s, const LinearPlan &pl, const void *q, const void *k,
                         const void *v, const float *eta, const float *w_init, void *out,
                         float *w_final, void *ws, hipStream_t stream);

// ---- LaCT SwiGLU ---------------------------------------------------------------
struct LactShape {
    int NH, Tq, Tkv, d, hid, chunk, loss, order, rownorm;
    int rule = 0;        // 0 gradient descent, 1 momentum, 2 Muon
    float beta = 0.f;    // momentum coefficient (rules 1, 2)
    int ns_steps = 0;    // Newton-Schulz steps (rule 2)
    float lr = 0.f;      // Muon step size (rule 2)
    // backward's forward replay: per chunk, the chunk-start weights and the
    // step direction ([chunk][NH][3][hid * d] fp32 each), or null
    float *save_w = nullptr, *save_d = nullptr;
};
struct LactPlan {
    int nchunks;
    int maxc;                 // tokens per chunk slot in the workspace
    size_t bytes;
    size_t off[16];
};
LactPlan lact_plan(const LactShape &s);
hipError_t lact_launch(const LactShape &s, const LactPlan &pl, const void *q, const void *k,
                       const void *v, const float *eta, const float *w1, const float *w2,
                       const float *w3, void *out, float *w1f, float *w2f, float *w3f, void *ws,
                       hipStream_t stream, hipStream_t aux, float *m1 = nullptr,
                       float *m2 = nullptr, float *m3 = nullptr);

// ---- LaCT SwiGLU backward (inner-product loss, gradient descent) --------------------
struct LactBwdPlan {
    LactPlan fwd;        // the replay's own workspace (at offset 0)
    int chunk, rpad;     // chunk length; rows of the per-token planes
    size_t o_save_w, o_save_d, o_wfin, o_lam, o_gam, o_wcb, o_f, o_e, o_dy, o_bdy, o_part;
    size_t bytes;
};
LactBwdPlan lact_bwd_plan(const LactShape &s);
hipError_t lact_bwd_launch(const LactShape &s, const LactBwdPlan &pl, const void *q, const void *k,
                           const void *v, const float *eta, const float *w1, const float *w2,
                           const float *w3, const void *dout, const float *dw1f, const float *dw2f,
                           const float *dw3f, void *dq, void *dk, void *dv, float *deta, float *dw1,
                           float *dw2, float *dw3, void *ws, hipStream_t stream);

// ---- decode steps (one token per head) ---------------------------------------------
hipError_t linear_decode_launch(int NH, int d, int bf16, int loss, const void *q, const void *k,
                                const void *v, const float *eta, float *w, float *anchor,
                                int anchor_update, void *out, hipStream_t stream);
size_t lact_decode_workspace(int NH, int hid);
hipError_t lact_decode_launch(int NH, int d, int hid, int bf16, const void *q, const float *w1,
                              const float *w2, const float *w3, void *out, void *ws,
                              hipStream_t stream);

// ---- sliding-window attention beside LaCT ------------------------------------------
hipError_t window_attn_launch(int NH, int T, int d, int window, float scale, int accumulate,
                              const void *q, const void *k, const void *v, void *out,
                              hipStream_t stream);

// ---- TTT-Linear backward (causal) -----------------------------------------------------
size_t linear_bwd_workspace(int NH, int Tkv, int d, int chunk);
hipError_t linear_bwd_launch(int NH, int Tq, int Tkv, int d, int chunk, int loss, int order,
                             int bf16, const void *q, const void *k, const void *v,
                             const float *eta, const float *w0, const void *dout, const float *dwf,
                             void *dq, void *dk, void *dv, float *deta, float *dw0, void *ws,
                             hipStream_t stream);
// chunks of several 16-token tiles (a separately compiled unit)
hipError_t linear_bwd_launch_tiled(int NH, int Tq, int Tkv, int d, int chunk, int loss, int order,
                                   int bf16, const void *q, const void *k, const void *v,
                                   const float *eta, const float *w0, const void *dout, const float *dwf,
                                   void *dq, void *dk, void *dv, float *deta, float *dw0, void *ws,
                                   hipStream_t stream);

}  // namespace tttk
