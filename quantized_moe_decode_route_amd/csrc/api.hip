// C ABI of libmoedec: argument validation and kernel launches.  Every entry
// point checks its arguments on the host before anything is enqueued, then
// enqueues its kernels on the caller's stream and returns without waiting.
#include <math.h>

#include "common.h"

#define MOEDEC_API extern "C" __attribute__((visibility("default")))

namespace moedec {
// quant.hip
hipError_t launch_quantize_rows(int bits, bool pack, const float* w, void* out, float* scales, int64_t rows,
                                int64_t row_len, hipStream_t stream);
}  // namespace moedec

using namespace moedec;

namespace {

constexpr int kAbiVersion = 2;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int device_status(hipError_t e) { return e == hipSuccess ? MOEDEC_OK : MOEDEC_ERR_DEVICE; }

// Checks shared by every call that touches the experts; fills `out`.
int check_experts(const moedec_experts* ex, const moedec_worklist* wl, int bits, int T, int top_k,
                  ExpertArgs& out) {
    if (!ex || !wl) return MOEDEC_ERR_INVALID_ARG;
    if (!wl->n_active || !wl->expert_id || !wl->seg || !wl->assign) return MOEDEC_ERR_INVALID_ARG;
    if (!ex->w_gate || !ex->w_up || !ex->w_down || !ex->s_gate || !ex->s_up || !ex->s_down)
        return MOEDEC_ERR_INVALID_ARG;
    if (ex->bits != bits) return MOEDEC_ERR_INVALID_ARG;
    if (T < 1 || top_k < 1 || ex->hidden < 1 || ex->inter < 1 || ex->n_experts < 1 || ex->n_shared < 0)
        return MOEDEC_ERR_INVALID_ARG;
    if (top_k > ex->n_experts) return MOEDEC_ERR_INVALID_ARG;
    const int cols_per_group = 128 / bits;     // columns in 16 bytes of codes
    if (ex->hidden % cols_per_group || ex->inter % cols_per_group) return MOEDEC_ERR_INVALID_ARG;
    if (T > MOEDEC_MAX_TOKENS || top_k > 32 || ex->n_shared > 8 || ex->n_experts > MOEDEC_MAX_EXPERTS ||
        ex->hidden > MOEDEC_MAX_DIM || ex->inter > MOEDEC_MAX_DIM)
        return MOEDEC_ERR_UNSUPPORTED;
    if (!aligned16(ex->w_gate) || !aligned16(ex->w_up) || !aligned16(ex->w_down)) return MOEDEC_ERR_INVALID_ARG;
    out.w_gate = ex->w_gate;
    out.w_up = ex->w_up;
    out.w_down = ex->w_down;
    out.s_gate = ex->s_gate;
    out.s_up = ex->s_up;
    out.s_down = ex->s_down;
    out.n_active = wl->n_active;
    out.expert_id = wl->expert_id;
    out.seg = wl->seg;
    out.assign = wl->assign;
    out.T = T;
    out.H = ex->hidden;
    out.I = ex->inter;
    out.top_k = top_k;
    out.slots = top_k + ex->n_shared;
    const int routed = ex->n_experts < T * top_k ? ex->n_experts : T * top_k;
    out.max_active = routed + ex->n_shared;
    return MOEDEC_OK;
}

int gate_up(int bits, const float* x, const moedec_experts* ex, const moedec_worklist* wl, int T, int top_k,
            float* h, void* stream) {
    if (!x || !h) return MOEDEC_ERR_INVALID_ARG;
    ExpertArgs a;
    const int st = check_experts(ex, wl, bits, T, top_k, a);
    if (st != MOEDEC_OK) return st;
    if (!aligned16(x)) return MOEDEC_ERR_INVALID_ARG;
    return device_status(launch_gate_up(bits, x, a, h, static_cast<hipStream_t>(stream)));
}

int down(int bits, const float* h, const moedec_experts* ex, const moedec_worklist* wl, const float* topk_w, int T,
         int top_k, float* y, void* stream) {
    if (!h || !topk_w || !y) return MOEDEC_ERR_INVALID_ARG;
    ExpertArgs a;
    const int st = check_experts(ex, wl, bits, T, top_k, a);
    if (st != MOEDEC_OK) return st;
    if (!aligned16(h)) return MOEDEC_ERR_INVALID_ARG;
    return device_status(launch_down(bits, h, topk_w, a, y, static_cast<hipStream_t>(stream)));
}

int down_em(int bits, const float* h, const moedec_experts* ex, const moedec_worklist* wl, const float* topk_w,
            const int32_t* topk_idx, int T, int top_k, float* part, float* y, void* stream) {
    if (!h || !topk_w || !y || !part) return MOEDEC_ERR_INVALID_ARG;
    ExpertArgs a;
    const int st = check_experts(ex, wl, bits, T, top_k, a);
    if (st != MOEDEC_OK) return st;
    if (!aligned16(h)) return MOEDEC_ERR_INVALID_ARG;
    return device_status(launch_down_em(bits, h, topk_w, topk_idx, a, part, y, static_cast<hipStream_t>(stream)));
}

int route_args_ok(int T, int H, int E, int n_group, int topk_group, int top_k, int n_shared, float rsf) {
    if (T < 1 || H < 4 || H % 4 || E < 2 || n_group < 1 || E % n_group || E / n_group < 2)
        return MOEDEC_ERR_INVALID_ARG;
    if (topk_group < 1 || topk_group > n_group || top_k < 1 || top_k > topk_group * (E / n_group))
        return MOEDEC_ERR_INVALID_ARG;
    if (n_shared < 0 || !isfinite(rsf)) return MOEDEC_ERR_INVALID_ARG;
    if (T > MOEDEC_MAX_TOKENS || E > MOEDEC_MAX_EXPERTS || n_group > 64 || top_k > 32 || n_shared > 8 ||
        H > MOEDEC_MAX_DIM)
        return MOEDEC_ERR_UNSUPPORTED;
    return MOEDEC_OK;
}

int layer_fused(int bits, const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                int T, int n_group, int topk_group, int top_k, float rsf, float top_p, float* x_out, float eps,
                float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl, float* h, float* y,
                int32_t* workspace, void* stream, int act8 = 0) {
    if (!x || !router_w || !bias || !scores || !topk_idx || !topk_w || !h || !y || !workspace)
        return MOEDEC_ERR_INVALID_ARG;
    if (isnan(top_p)) return MOEDEC_ERR_INVALID_ARG;
    if (x_out && !(eps >= 0.0f && isfinite(eps))) return MOEDEC_ERR_INVALID_ARG;
    FusedLayerArgs f{};
    int st = check_experts(ex, wl, bits, T, top_k, f.ex);
    if (st != MOEDEC_OK) return st;
    st = route_args_ok(T, ex->hidden, ex->n_experts, n_group, topk_group, top_k, ex->n_shared, rsf);
    if (st != MOEDEC_OK) return st;
    if (!aligned16(x) || !aligned16(router_w) || !aligned16(h) || (reinterpret_cast<uintptr_t>(workspace) & 7u))
        return MOEDEC_ERR_INVALID_ARG;
    if (T > MOEDEC_FUSED_MAX_TOKENS || ex->n_experts > MOEDEC_FUSED_MAX_EXPERTS) return MOEDEC_ERR_UNSUPPORTED;
    f.x = x;
    f.router_w = router_w;
    f.bias = bias;
    f.scores = scores;
    f.topk_idx = topk_idx;
    f.topk_w = topk_w;
    f.wl_n_active = wl->n_active;
    f.wl_expert_id = wl->expert_id;
    f.wl_seg = wl->seg;
    f.wl_assign = wl->assign;
    f.h = h;
    f.y = y;
    f.workspace = workspace;
    f.T = T;
    f.E = ex->n_experts;
    f.n_group = n_group;
    f.topk_group = topk_group;
    f.n_shared = ex->n_shared;
    f.rsf = rsf;
    f.top_p = top_p;
    f.x_out = x_out;
    f.eps = eps;
    f.act8 = act8;
    const hipError_t err = act8 ? launch_layer_fused(bits, f, static_cast<hipStream_t>(stream))
                                : launch_layer_pipe(bits, f, static_cast<hipStream_t>(stream));
    if (err == hipErrorInvalidValue) return MOEDEC_ERR_UNSUPPORTED;   // shapes the LDS plan cannot hold
    return device_status(err);
}

int pack(int bits, const int8_t* codes, uint8_t* packed, int64_t rows, int64_t row_len, void* stream) {
    if (rows < 0 || row_len < 0 || row_len % (8 / bits)) return MOEDEC_ERR_INVALID_ARG;
    if (rows * row_len == 0) return MOEDEC_OK;
    if (!codes || !packed) return MOEDEC_ERR_INVALID_ARG;
    return device_status(launch_pack(bits, codes, packed, rows, row_len, static_cast<hipStream_t>(stream)));
}

int unpack(int bits, const uint8_t* packed, int8_t* codes, int64_t rows, int64_t row_len, void* stream) {
    if (rows < 0 || row_len < 0 || row_len % (8 / bits)) return MOEDEC_ERR_INVALID_ARG;
    if (rows * row_len == 0) return MOEDEC_OK;
    if (!codes || !packed) return MOEDEC_ERR_INVALID_ARG;
    return device_status(launch_unpack(bits, packed, codes, rows, row_len, static_cast<hipStream_t>(stream)));
}

int quantize(int bits, bool pack, const float* w, void* out, float* scales, int64_t rows, int64_t row_len,
             void* stream) {
    if (rows < 0 || row_len < 0 || row_len % 4) return MOEDEC_ERR_INVALID_ARG;
    if (rows == 0) return MOEDEC_OK;
    if (!scales || (row_len > 0 && (!w || !out))) return MOEDEC_ERR_INVALID_ARG;
    const uintptr_t out_align = (!pack || bits == 8) ? 4 : bits == 4 ? 2 : 1;
    if (!aligned16(w) || (reinterpret_cast<uintptr_t>(scales) & 3u) ||
        (reinterpret_cast<uintptr_t>(out) & (out_align - 1)))
        return MOEDEC_ERR_INVALID_ARG;
    if (rows > 0x7FFFFFFF) return MOEDEC_ERR_UNSUPPORTED;              // one workgroup per row
    return device_status(launch_quantize_rows(bits, pack, w, out, scales, rows, row_len,
                                              static_cast<hipStream_t>(stream)));
}

}  // namespace

MOEDEC_API const char* moedec_status_string(int status) {
    switch (status) {
        case MOEDEC_OK: return "ok";
        case MOEDEC_ERR_INVALID_ARG: return "invalid argument";
        case MOEDEC_ERR_UNSUPPORTED: return "unsupported shape or size";
        case MOEDEC_ERR_DEVICE: return "device launch error";
        default: return "unknown status";
    }
}

MOEDEC_API int moedec_abi_version(void) { return kAbiVersion; }

namespace {
int route(const float* x, const float* router_w, const float* bias, int T, int H, int E, int n_group,
          int topk_group, int top_k, int n_shared, float rsf, float top_p, float* scores, int32_t* topk_idx,
          float* topk_w, const moedec_worklist* wl, void* stream) {
    if (!x || !router_w || !bias || !scores || !topk_idx || !topk_w) return MOEDEC_ERR_INVALID_ARG;
    if (wl && (!wl->n_active || !wl->expert_id || !wl->seg || !wl->assign)) return MOEDEC_ERR_INVALID_ARG;
    if (isnan(top_p)) return MOEDEC_ERR_INVALID_ARG;
    const int st = route_args_ok(T, H, E, n_group, topk_group, top_k, n_shared, rsf);
    if (st != MOEDEC_OK) return st;
    if (!aligned16(x) || !aligned16(router_w)) return MOEDEC_ERR_INVALID_ARG;
    return device_status(launch_route(x, router_w, bias, T, H, E, n_group, topk_group, top_k, n_shared, rsf, top_p,
                                      scores, topk_idx, topk_w, wl, static_cast<hipStream_t>(stream)));
}
}  // namespace

MOEDEC_API int moe_route_topk(const float* x, const float* router_w, const float* bias, int T, int H, int E,
                              int n_group, int topk_group, int top_k, int n_shared, float routed_scaling_factor,
                              float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                              void* stream) {
    return route(x, router_w, bias, T, H, E, n_group, topk_group, top_k, n_shared, routed_scaling_factor, 1.0f,
                 scores, topk_idx, topk_w, wl, stream);
}

MOEDEC_API int moe_route_topp(const float* x, const float* router_w, const float* bias, int T, int H, int E,
                              int n_group, int topk_group, int top_k, int n_shared, float routed_scaling_factor,
                              float top_p, float* scores, int32_t* topk_idx, float* topk_w,
                              const moedec_worklist* wl, void* stream) {
    return route(x, router_w, bias, T, H, E, n_group, topk_group, top_k, n_shared, routed_scaling_factor, top_p,
                 scores, topk_idx, topk_w, wl, stream);
}

MOEDEC_API int moe_expert_gate_up_silu_q4(const float* x, const moedec_experts* ex, const moedec_worklist* wl,
                                          int T, int top_k, float* h, void* stream) {
    return gate_up(4, x, ex, wl, T, top_k, h, stream);
}
MOEDEC_API int moe_expert_gate_up_silu_q8(const float* x, const moedec_experts* ex, const moedec_worklist* wl,
                                          int T, int top_k, float* h, void* stream) {
    return gate_up(8, x, ex, wl, T, top_k, h, stream);
}
MOEDEC_API int moe_expert_gate_up_silu_q2(const float* x, const moedec_experts* ex, const moedec_worklist* wl,
                                          int T, int top_k, float* h, void* stream) {
    return gate_up(2, x, ex, wl, T, top_k, h, stream);
}

MOEDEC_API int moe_expert_down_combine_em_q4(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                                             const float* topk_w, const int32_t* topk_idx, int T, int top_k,
                                             float* part, float* y, void* stream) {
    return down_em(4, h, ex, wl, topk_w, topk_idx, T, top_k, part, y, stream);
}
MOEDEC_API int moe_expert_down_combine_em_noalloc_q4(const float* h, const moedec_experts* ex,
                                                     const moedec_worklist* wl, const float* topk_w,
                                                     const int32_t* topk_idx, int T, int top_k, float* y,
                                                     void* stream) {
    if (!h || !topk_w || !y) return MOEDEC_ERR_INVALID_ARG;
    ExpertArgs a;
    const int st = check_experts(ex, wl, 4, T, top_k, a);
    if (st != MOEDEC_OK) return st;
    if (!aligned16(h)) return MOEDEC_ERR_INVALID_ARG;
    if ((long long)a.T * a.slots * a.H > MOEDEC_NOALLOC_PART_FLOATS) return MOEDEC_ERR_UNSUPPORTED;
    return device_status(launch_down_em_noalloc(4, h, topk_w, topk_idx, a, y, static_cast<hipStream_t>(stream)));
}
MOEDEC_API int moe_expert_down_combine_q4(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                                          const float* topk_w, int T, int top_k, float* y, void* stream) {
    return down(4, h, ex, wl, topk_w, T, top_k, y, stream);
}
MOEDEC_API int moe_expert_down_combine_em_q8(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                                             const float* topk_w, const int32_t* topk_idx, int T, int top_k,
                                             float* part, float* y, void* stream) {
    return down_em(8, h, ex, wl, topk_w, topk_idx, T, top_k, part, y, stream);
}
MOEDEC_API int moe_expert_down_combine_q8(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                                          const float* topk_w, int T, int top_k, float* y, void* stream) {
    return down(8, h, ex, wl, topk_w, T, top_k, y, stream);
}
MOEDEC_API int moe_expert_down_combine_em_q2(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                                             const float* topk_w, const int32_t* topk_idx, int T, int top_k,
                                             float* part, float* y, void* stream) {
    return down_em(2, h, ex, wl, topk_w, topk_idx, T, top_k, part, y, stream);
}
MOEDEC_API int moe_expert_down_combine_q2(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                                          const float* topk_w, int T, int top_k, float* y, void* stream) {
    return down(2, h, ex, wl, topk_w, T, top_k, y, stream);
}

MOEDEC_API int moe_pack_q4(const int8_t* codes, uint8_t* packed, int64_t rows, int64_t row_len, void* stream) {
    return pack(4, codes, packed, rows, row_len, stream);
}
MOEDEC_API int moe_unpack_q4(const uint8_t* packed, int8_t* codes, int64_t rows, int64_t row_len, void* stream) {
    return unpack(4, packed, codes, rows, row_len, stream);
}
MOEDEC_API int moe_pack_q8(const int8_t* codes, uint8_t* packed, int64_t rows, int64_t row_len, void* stream) {
    return pack(8, codes, packed, rows, row_len, stream);
}
MOEDEC_API int moe_unpack_q8(const uint8_t* packed, int8_t* codes, int64_t rows, int64_t row_len, void* stream) {
    return unpack(8, packed, codes, rows, row_len, stream);
}
MOEDEC_API int moe_pack_q2(const int8_t* codes, uint8_t* packed, int64_t rows, int64_t row_len, void* stream) {
    return pack(2, codes, packed, rows, row_len, stream);
}
MOEDEC_API int moe_unpack_q2(const uint8_t* packed, int8_t* codes, int64_t rows, int64_t row_len, void* stream) {
    return unpack(2, packed, codes, rows, row_len, stream);
}

MOEDEC_API int moe_quantize_rows_q8(const float* w, int8_t* codes, float* scales, int64_t rows, int64_t row_len,
                                    void* stream) {
    return quantize(8, false, w, codes, scales, rows, row_len, stream);
}
MOEDEC_API int moe_quantize_rows_q4(const float* w, int8_t* codes, float* scales, int64_t rows, int64_t row_len,
                                    void* stream) {
    return quantize(4, false, w, codes, scales, rows, row_len, stream);
}
MOEDEC_API int moe_quantize_rows_q2(const float* w, int8_t* codes, float* scales, int64_t rows, int64_t row_len,
                                    void* stream) {
    return quantize(2, false, w, codes, scales, rows, row_len, stream);
}
MOEDEC_API int moe_quantize_pack_rows_q8(const float* w, uint8_t* packed, float* scales, int64_t rows,
                                         int64_t row_len, void* stream) {
    return quantize(8, true, w, packed, scales, rows, row_len, stream);
}
MOEDEC_API int moe_quantize_pack_rows_q4(const float* w, uint8_t* packed, float* scales, int64_t rows,
                                         int64_t row_len, void* stream) {
    return quantize(4, true, w, packed, scales, rows, row_len, stream);
}
MOEDEC_API int moe_quantize_pack_rows_q2(const float* w, uint8_t* packed, float* scales, int64_t rows,
                                         int64_t row_len, void* stream) {
    return quantize(2, true, w, packed, scales, rows, row_len, stream);
}

MOEDEC_API int moe_residual_rmsnorm(float* x, const float* y, float* xn, int T, int H, float eps, void* stream) {
    if (!x || !xn || T < 1 || H < 1 || !(eps >= 0.0f)) return MOEDEC_ERR_INVALID_ARG;
    return device_status(launch_residual_rmsnorm(x, y, xn, T, H, eps, static_cast<hipStream_t>(stream)));
}

MOEDEC_API int moe_layer_fused_q4(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                                  int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                                  float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                                  float* h, float* y, int32_t* workspace, void* stream) {
    return layer_fused(4, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, 1.0f,
                       nullptr, 0.0f, scores, topk_idx, topk_w, wl, h, y, workspace, stream);
}
MOEDEC_API int moe_layer_fused_topp_q4(const float* x, const float* router_w, const float* bias,
                                       const moedec_experts* ex, int T, int n_group, int topk_group, int top_k,
                                       float routed_scaling_factor, float top_p, float* scores, int32_t* topk_idx,
                                       float* topk_w, const moedec_worklist* wl, float* h, float* y,
                                       int32_t* workspace, void* stream) {
    return layer_fused(4, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, top_p,
                       nullptr, 0.0f, scores, topk_idx, topk_w, wl, h, y, workspace, stream);
}
MOEDEC_API int moe_layer_fused_act8_q4(const float* x, const float* router_w, const float* bias,
                                       const moedec_experts* ex, int T, int n_group, int topk_group, int top_k,
                                       float routed_scaling_factor, float top_p, float* scores, int32_t* topk_idx,
                                       float* topk_w, const moedec_worklist* wl, float* h, float* y,
                                       int32_t* workspace, void* stream) {
    return layer_fused(4, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, top_p,
                       nullptr, 0.0f, scores, topk_idx, topk_w, wl, h, y, workspace, stream, 1);
}
MOEDEC_API int moe_layer_fused_resid_q4(const float* x, const float* router_w, const float* bias,
                                        const moedec_experts* ex, int T, int n_group, int topk_group, int top_k,
                                        float routed_scaling_factor, float top_p, float eps, float* x_out,
                                        float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                                        float* h, float* y, int32_t* workspace, void* stream) {
    if (!x_out) return MOEDEC_ERR_INVALID_ARG;
    return layer_fused(4, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, top_p,
                       x_out, eps, scores, topk_idx, topk_w, wl, h, y, workspace, stream);
}
MOEDEC_API int moe_layer_fused_q8(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                                  int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                                  float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                                  float* h, float* y, int32_t* workspace, void* stream) {
    return layer_fused(8, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, 1.0f,
                       nullptr, 0.0f, scores, topk_idx, topk_w, wl, h, y, workspace, stream);
}
MOEDEC_API int moe_layer_fused_topp_q8(const float* x, const float* router_w, const float* bias,
                                       const moedec_experts* ex, int T, int n_group, int topk_group, int top_k,
                                       float routed_scaling_factor, float top_p, float* scores, int32_t* topk_idx,
                                       float* topk_w, const moedec_worklist* wl, float* h, float* y,
                                       int32_t* workspace, void* stream) {
    return layer_fused(8, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, top_p,
                       nullptr, 0.0f, scores, topk_idx, topk_w, wl, h, y, workspace, stream);
}
MOEDEC_API int moe_layer_fused_act8_q8(const float* x, const float* router_w, const float* bias,
                                       const moedec_experts* ex, int T, int n_group, int topk_group, int top_k,
                                       float routed_scaling_factor, float top_p, float* scores, int32_t* topk_idx,
                                       float* topk_w, const moedec_worklist* wl, float* h, float* y,
                                       int32_t* workspace, void* stream) {
    return layer_fused(8, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, top_p,
                       nullptr, 0.0f, scores, topk_idx, topk_w, wl, h, y, workspace, stream, 1);
}
MOEDEC_API int moe_layer_fused_resid_q8(const float* x, const float* router_w, const float* bias,
                                        const moedec_experts* ex, int T, int n_group, int topk_group, int top_k,
                                        float routed_scaling_factor, float top_p, float eps, float* x_out,
                                        float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                                        float* h, float* y, int32_t* workspace, void* stream) {
    if (!x_out) return MOEDEC_ERR_INVALID_ARG;
    return layer_fused(8, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, top_p,
                       x_out, eps, scores, topk_idx, topk_w, wl, h, y, workspace, stream);
}
MOEDEC_API int moe_layer_fused_q2(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                                  int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                                  float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                                  float* h, float* y, int32_t* workspace, void* stream) {
    return layer_fused(2, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, 1.0f,
                       nullptr, 0.0f, scores, topk_idx, topk_w, wl, h, y, workspace, stream);
}
MOEDEC_API int moe_layer_fused_topp_q2(const float* x, const float* router_w, const float* bias,
                                       const moedec_experts* ex, int T, int n_group, int topk_group, int top_k,
                                       float routed_scaling_factor, float top_p, float* scores, int32_t* topk_idx,
                                       float* topk_w, const moedec_worklist* wl, float* h, float* y,
                                       int32_t* workspace, void* stream) {
    return layer_fused(2, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, top_p,
                       nullptr, 0.0f, scores, topk_idx, topk_w, wl, h, y, workspace, stream);
}
MOEDEC_API int moe_layer_fused_act8_q2(const float* x, const float* router_w, const float* bias,
                                       const moedec_experts* ex, int T, int n_group, int topk_group, int top_k,
                                       float routed_scaling_factor, float top_p, float* scores, int32_t* topk_idx,
                                       float* topk_w, const moedec_worklist* wl, float* h, float* y,
                                       int32_t* workspace, void* stream) {
    return layer_fused(2, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, top_p,
                       nullptr, 0.0f, scores, topk_idx, topk_w, wl, h, y, workspace, stream, 1);
}
MOEDEC_API int moe_layer_fused_resid_q2(const float* x, const float* router_w, const float* bias,
                                        const moedec_experts* ex, int T, int n_group, int topk_group, int top_k,
                                        float routed_scaling_factor, float top_p, float eps, float* x_out,
                                        float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                                        float* h, float* y, int32_t* workspace, void* stream) {
    if (!x_out) return MOEDEC_ERR_INVALID_ARG;
    return layer_fused(2, x, router_w, bias, ex, T, n_group, topk_group, top_k, routed_scaling_factor, top_p,
                       x_out, eps, scores, topk_idx, topk_w, wl, h, y, workspace, stream);
}
