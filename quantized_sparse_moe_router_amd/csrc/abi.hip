// abi.hip -- the library's C entry points: argument validation, workspace sizing and
// shape-based dispatch to the gfx950 kernels.  See include/moe.h for the contract.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "moe_common.h"

// Workspace of moe_layer_decode_noalloc: one copy per GPU, held until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host the name is a
// stand-in, not a device address); it passes the address hipGetSymbolAddress returns
// for the current device (scratch_base below).
constexpr size_t kNoAllocScratchBytes = 512 * 1024;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

moe_status ok() {
    g_last_error.clear();
    return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round_up(size_t n) { return (n + 255) & ~size_t(255); }

bool supported_ffn_dim(int n) {
    return n == 128 || n == 256 || n == 512 || n == 1024 || n == 2048 || n == 4096;
}

bool supported_router_dim(int fmt, int d) {
    if (fmt == MOE_FMT_FP32) return d == 256 || d == 512 || d == 1024 || d == 2048 || d == 4096;
    return d == 1024 || d == 2048 || d == 4096;
}

constexpr int kMaxExperts = 1024;   // the decode layer's selection holds <= 16 keys per lane
constexpr int kMaxK = 64;
constexpr int64_t kDecodeMaxPairs = 64; // pairs up to which moe_layer_decode runs

// route workspace, exact form: [counter][logits]
size_t route_exact_ws(int64_t T, int E) {
    return moe::kRouteCounterBytes + round_up((size_t)T * (size_t)E * sizeof(float));
}

// the bounded form (many tokens, no logits wanted) runs when this holds
bool route_bounded(int64_t T, const float* logits) {
    return logits == nullptr && T > moe::kRouteSplitMaxTokens;
}

// route workspace: [counter]; with no logits from the caller also [logits], and for the
// bounded form [plane rows][row norm bounds]
size_t route_ws(int64_t T, int E, int d, bool need_logits) {
    if (!need_logits) return moe::kRouteCounterBytes;
    size_t n = route_exact_ws(T, E);
    if (route_bounded(T, nullptr))
        n += round_up(moe::route_bounded_planes_bytes(E, d)) + round_up((size_t)E * sizeof(float));
    return n;
}

// expert FFN workspace: GEMV [h], or in sorted mode [h][chunk list][GEMM work list][count];
// MFMA [h][tile list][count]
size_t ffn_ws(int64_t rows, int E, int F) {
    size_t gemv = round_up((size_t)rows * (size_t)F * 2);
    if (rows > moe::kGemvMaxBallotPairs) gemv = moe::gemv_sorted_ws_layout(rows, E, F).bytes;
    const size_t mfma = moe::ffn_mfma_ws_bytes(rows, E, F);
    return gemv > mfma ? gemv : mfma;
}

// decode layer workspace: [route workspace: counter, logits [T][E] fp32][h rows of every
// slot]
size_t decode_ws(int T, int k, int E, int d, int F) {
    return round_up(route_exact_ws(T, E)) + moe::decode_ws_layout(T, k, d, F).bytes;
}

// the decode operations run for these sizes: at most 64 pairs, the h rows of every slot
// within LDS, and a (d_model, d_ff) pair with decode kernels
bool decode_runs(int T, int k, int d, int F) {
    return d > 0 && F > 0 && (int64_t)T * k <= kDecodeMaxPairs && moe::ffn_gemv_has_shape(d, F) &&
           moe::decode_fits(T, k, F, false);
}

// decode block workspace: the decode layer's, then xn [T][d] bf16 and z [T] fp32
size_t block_ws(int T, int k, int E, int d, int F) {
    return decode_ws(T, k, E, d, F) + round_up((size_t)T * d * 2) + round_up((size_t)T * 4);
}

bool finite_f32(float v) { return v == v && v - v == 0.0f; }

// moe_norm checks shared by moe_rmsnorm and moe_block_decode
moe_status check_norm(const moe_norm* n, int d, const char* who) {
    if (!n) return fail(MOE_ERR_INVALID_ARG, "%s: norm descriptor is NULL", who);
    if (!n->gamma || !aligned16(n->gamma))
        return fail(MOE_ERR_INVALID_ARG, "%s: gamma NULL or not 16-byte aligned", who);
    if (n->gate_w && !aligned16(n->gate_w))
        return fail(MOE_ERR_INVALID_ARG, "%s: gate_w not 16-byte aligned", who);
    if (!finite_f32(n->eps) || n->eps < 0.0f || !finite_f32(n->gate_b))
        return fail(MOE_ERR_INVALID_ARG, "%s: eps must be finite and >= 0, gate_b finite", who);
    if (d != 256 && d != 512 && d != 1024 && d != 2048 && d != 4096)
        return fail(MOE_ERR_INVALID_ARG, "%s: d_model %d must be 256..4096, a power of two",
                    who, d);
    return MOE_OK;
}

// Router descriptor checks shared by moe_route and moe_layer_decode.
moe_status check_router(const moe_router* r, const char* who) {
    if (!r) return fail(MOE_ERR_INVALID_ARG, "%s: router descriptor is NULL", who);
    if (r->fmt != MOE_FMT_FP32 && r->fmt != MOE_FMT_INT8_ROW)
        return fail(MOE_ERR_INVALID_ARG, "%s: router format %d is not FP32 or INT8_ROW", who,
                    r->fmt);
    if (r->reserved != 0) return fail(MOE_ERR_INVALID_ARG, "%s: reserved field not 0", who);
    const int E = r->n_experts, d = r->d_model;
    if (E < 1 || E > kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "%s: n_experts %d outside [1, %d]", who, E,
                    kMaxExperts);
    if (!supported_router_dim(r->fmt, d))
        return fail(MOE_ERR_INVALID_ARG,
                    "%s: d_model %d unsupported (FP32: 256..4096 powers of two; "
                    "INT8_ROW: 1024, 2048, 4096)", who, d);
    if (!r->w || !aligned16(r->w))
        return fail(MOE_ERR_INVALID_ARG, "%s: router weights NULL or not 16-byte aligned", who);
    if (r->fmt == MOE_FMT_INT8_ROW && !r->scale)
        return fail(MOE_ERR_INVALID_ARG, "%s: INT8_ROW router needs scales", who);
    return MOE_OK;
}

bool expert_fmt(int fmt) {
    return fmt == MOE_FMT_INT4_G32 || fmt == MOE_FMT_INT6_G32 || fmt == MOE_FMT_INT3_G32 ||
           fmt == MOE_FMT_INT2_G32;
}

// Expert-set descriptor checks shared by moe_expert_ffn and moe_layer_decode.
moe_status check_experts(const moe_experts* ex, const char* who) {
    if (!ex) return fail(MOE_ERR_INVALID_ARG, "%s: expert descriptor is NULL", who);
    if (!expert_fmt(ex->fmt))
        return fail(MOE_ERR_INVALID_ARG,
                    "%s: format %d is not INT4_G32/INT6_G32/INT3_G32/INT2_G32", who, ex->fmt);
    const int E = ex->n_experts, d = ex->d_model, F = ex->d_ff;
    if (E < 1 || E > kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "%s: n_experts %d", who, E);
    if (!supported_ffn_dim(d) || d < 256 || !supported_ffn_dim(F))
        return fail(MOE_ERR_INVALID_ARG,
                    "%s: d_model %d must be 256..4096 and d_ff %d 128..4096, "
                    "powers of two", who, d, F);
    if (!ex->w_gate || !ex->w_up || !ex->w_down || !ex->s_gate || !ex->s_up || !ex->s_down)
        return fail(MOE_ERR_INVALID_ARG, "%s: a weight or scale pointer is NULL", who);
    if (!aligned16(ex->w_gate) || !aligned16(ex->w_up) || !aligned16(ex->w_down) ||
        !aligned16(ex->s_gate) || !aligned16(ex->s_up) || !aligned16(ex->s_down))
        return fail(MOE_ERR_INVALID_ARG, "%s: weights or scales not 16-byte aligned", who);
    return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_DEVICE: return "device reported bad data";
        default: return "unknown status";
    }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_workspace_size(int32_t op, int32_t T, int32_t k, int32_t E, int32_t d,
                          int32_t d_ff) {
    // 0 for sizes every call of these operations rejects; within these limits no product
    // below exceeds 2^63
    if (T <= 0 || k <= 0 || E <= 0 || E > kMaxExperts) return 0;
    const int64_t pairs = (int64_t)T * k;
    if (pairs > INT32_MAX) return 0;
    switch (op) {
        case MOE_OP_ROUTE:
            // the bounded form keeps bf16 copies of the router rows: d must be a size
            if (route_bounded(T, nullptr) && d <= 0) return 0;
            return route_ws(T, E, d, true);
        case MOE_OP_PERMUTE: return moe::permute_ws_bytes(pairs, E);
        case MOE_OP_EXPERT_FFN: return d_ff > 0 ? ffn_ws(pairs, E, d_ff) : 0;
        // the decode operations: 0 also where they do not run (more than 64 pairs, h rows
        // beyond LDS, a (d_model, d_ff) pair without decode kernels)
        case MOE_OP_LAYER_DECODE:
            return decode_runs(T, k, d, d_ff) ? decode_ws(T, k, E, d, d_ff) : 0;
        case MOE_OP_EXPERTS_DECODE:
            return decode_runs(T, k, d, d_ff) ? moe::decode_ws_layout(T, k, d, d_ff).bytes : 0;
        case MOE_OP_BLOCK_DECODE:
            return decode_runs(T, k, d, d_ff) ? block_ws(T, k, E, d, d_ff) : 0;
        default: return 0;
    }
}

moe_status moe_route(const moe_router* r, const uint16_t* x, int32_t T, int32_t k,
                     int32_t* ids, float* weights, float* logits, void* ws, size_t ws_bytes,
                     void* stream) {
    const moe_status st = check_router(r, "moe_route");
    if (st != MOE_OK) return st;
    const int E = r->n_experts;
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_route: T = %d < 0", T);
    if (k < 1 || k > E || k > kMaxK)
        return fail(MOE_ERR_INVALID_ARG, "moe_route: k = %d outside [1, min(E, %d)]", k, kMaxK);
    if (T == 0) return ok();
    if (!x || !aligned16(x))
        return fail(MOE_ERR_INVALID_ARG, "moe_route: x NULL or not 16-byte aligned");
    if (!ids || !weights) return fail(MOE_ERR_INVALID_ARG, "moe_route: ids/weights NULL");
    const size_t need = route_ws(T, E, r->d_model, logits == nullptr);
    if (!ws || ws_bytes < need || !aligned16(ws))
        return fail(MOE_ERR_WORKSPACE,
                    "moe_route: needs a 16-byte aligned workspace of %zu bytes (got %zu)", need,
                    ws_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* base = static_cast<uint8_t*>(ws);
    unsigned* counter = reinterpret_cast<unsigned*>(base);
    float* lg = logits ? logits : reinterpret_cast<float*>(base + moe::kRouteCounterBytes);
    if (route_bounded(T, logits)) {
        uint8_t* p = base + route_exact_ws(T, E);
        uint16_t* planes = reinterpret_cast<uint16_t*>(p);
        float* nw = reinterpret_cast<float*>(
            p + round_up(moe::route_bounded_planes_bytes(E, r->d_model)));
        hipError_t e = moe::launch_route_bounded_logits(*r, x, T, planes, nw, lg, s);
        if (e != hipSuccess) return hip_status(e, "moe_route: bounded logits");
        return hip_status(moe::launch_route_bounded_select(*r, x, T, k, nw, lg, ids, weights, s),
                          "moe_route: selection");
    }
    return hip_status(moe::launch_route(*r, x, T, k, ids, weights, lg, counter, s),
                      "moe_route");
}

moe_status moe_permute(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t* offsets,
                       int32_t* sorted_pairs, int32_t* pair_pos, void* ws, size_t ws_bytes,
                       void* stream) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_permute: T = %d < 0", T);
    if (k < 1 || k > kMaxK) return fail(MOE_ERR_INVALID_ARG, "moe_permute: k = %d", k);
    if (E < 1 || E > kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "moe_permute: E = %d outside [1, %d]", E, kMaxExperts);
    if ((int64_t)T * k > INT32_MAX)
        return fail(MOE_ERR_INVALID_ARG, "moe_permute: T*k overflows int32");
    if (!offsets) return fail(MOE_ERR_INVALID_ARG, "moe_permute: offsets NULL");
    if (T > 0 && (!ids || !sorted_pairs || !pair_pos))
        return fail(MOE_ERR_INVALID_ARG, "moe_permute: ids/sorted_pairs/pair_pos NULL");
    const size_t need = moe::permute_ws_bytes((int64_t)T * k, E);
    if (need && (!ws || ws_bytes < need || !aligned16(ws)))
        return fail(MOE_ERR_WORKSPACE, "moe_permute: needs %zu workspace bytes (got %zu)", need,
                    ws_bytes);
    return hip_status(moe::launch_permute(ids, T, k, E, offsets, sorted_pairs, pair_pos, ws,
                                          static_cast<hipStream_t>(stream)),
                      "moe_permute");
}

moe_status moe_expert_ffn(const moe_experts* ex, const uint16_t* x, int32_t T, int32_t k,
                          const int32_t* ids, const int32_t* offsets,
                          const int32_t* sorted_pairs, uint16_t* y, void* ws,
                          size_t ws_bytes, void* stream) {
    const moe_status st = check_experts(ex, "moe_expert_ffn");
    if (st != MOE_OK) return st;
    const int E = ex->n_experts, d = ex->d_model, F = ex->d_ff;
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: T = %d < 0", T);
    const bool grouped = ids || offsets || sorted_pairs;
    if (grouped && (!ids || !offsets || !sorted_pairs))
        return fail(MOE_ERR_INVALID_ARG,
                    "moe_expert_ffn: ids, offsets and sorted_pairs must be all set or all NULL");
    if (!grouped && E != 1)
        return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: dense mode needs n_experts == 1");
    if (grouped && (k < 1 || k > kMaxK))
        return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: k = %d", k);
    if (T == 0) return ok();
    if (!x || !aligned16(x) || !y || !aligned16(y))
        return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: x/y NULL or not 16-byte aligned");
    const int64_t rows = grouped ? (int64_t)T * k : (int64_t)T;
    if (rows > INT32_MAX) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: too many rows");
    const size_t need = ffn_ws(rows, grouped ? E : 1, F);
    if (!ws || ws_bytes < need || !aligned16(ws))
        return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn: needs %zu workspace bytes (got %zu)",
                    need, ws_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the GEMV for every call of its shapes up to 64 rows and for every grouped call (from
    // kHybridMinRows rows only the experts with few pairs, the others on the grouped GEMM)
    const bool gemv = moe::ffn_gemv_has_shape(d, F) &&
                      (rows <= moe::kGemvMaxBallotRows || grouped);
    // the grouped GEMM addresses x and h rows with 32-bit byte offsets
    if ((!gemv || (grouped && rows >= moe::kHybridMinRows)) &&
        ((uint64_t)T * (uint64_t)d * 2 >= (1ull << 32) ||
         (uint64_t)rows * (uint64_t)F * 2 >= (1ull << 32)))
        return fail(MOE_ERR_UNSUPPORTED,
                    "moe_expert_ffn: x (T*d_model) and h (rows*d_ff) must each be under "
                    "4 GiB of bf16; split the call");
    const hipError_t e =
        gemv ? moe::launch_ffn_gemv(*ex, x, T, grouped ? k : 1, ids, offsets, sorted_pairs, y,
                                    ws, s)
             : moe::launch_ffn_mfma(*ex, x, T, grouped ? k : 1, offsets, sorted_pairs, y, ws,
                                    s);
    return hip_status(e, "moe_expert_ffn");
}

moe_status moe_combine(const uint16_t* y_pairs, const int32_t* pair_pos, const float* weights,
                       const uint16_t* y_shared, const uint16_t* residual, int32_t T, int32_t k,
                       int32_t d, uint16_t* out, void* stream) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_combine: T = %d < 0", T);
    if (k < 1 || k > kMaxK) return fail(MOE_ERR_INVALID_ARG, "moe_combine: k = %d", k);
    if (d < 8 || d % 8 != 0) return fail(MOE_ERR_INVALID_ARG, "moe_combine: d = %d", d);
    if (T == 0) return ok();
    if (!y_pairs || !pair_pos || !weights || !out)
        return fail(MOE_ERR_INVALID_ARG, "moe_combine: y_pairs/pair_pos/weights/out NULL");
    if (!aligned16(y_pairs) || !aligned16(out) || (y_shared && !aligned16(y_shared)) ||
        (residual && !aligned16(residual)))
        return fail(MOE_ERR_INVALID_ARG, "moe_combine: bf16 rows must be 16-byte aligned");
    return hip_status(moe::launch_combine(y_pairs, pair_pos, weights, y_shared, residual,
                                          nullptr, T, k,
                                          d, out, static_cast<hipStream_t>(stream)),
                      "moe_combine");
}

}  // extern "C"

namespace {

// Checks shared by moe_experts_decode and moe_layer_decode (routed, shared, T, k, rows).
moe_status check_decode(const moe_experts* routed, const moe_experts* shared, int T, int k,
                        const uint16_t* x, const uint16_t* residual, const uint16_t* out,
                        const char* who) {
    moe_status st = check_experts(routed, who);
    if (st != MOE_OK) return st;
    const int E = routed->n_experts, d = routed->d_model, F = routed->d_ff;
    if (shared) {
        st = check_experts(shared, who);
        if (st != MOE_OK) return st;
        if (shared->n_experts != 1)
            return fail(MOE_ERR_INVALID_ARG, "%s: shared set must have 1 expert", who);
        if (shared->fmt != routed->fmt || shared->d_model != d || shared->d_ff != F)
            return fail(MOE_ERR_UNSUPPORTED,
                        "%s: the shared expert must have the routed experts' format and shape",
                        who);
    }
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T = %d < 0", who, T);
    if (k < 1 || k > E || k > kMaxK)
        return fail(MOE_ERR_INVALID_ARG, "%s: k = %d outside [1, min(E, %d)]", who, k, kMaxK);
    if (T == 0) return MOE_OK;
    if ((int64_t)T * k > kDecodeMaxPairs || !moe::ffn_gemv_has_shape(d, F) ||
        !moe::decode_fits(T, k, F, shared != nullptr))
        return fail(MOE_ERR_UNSUPPORTED,
                    "%s: T*k = %d (at most %d; h rows of all slots within %d KiB) or shape "
                    "(%d, %d) not supported; use the four calls", who, T * k,
                    (int)kDecodeMaxPairs, (int)(moe::kDecodeMaxLds / 1024), d, F);
    if (!x || !aligned16(x) || !out || !aligned16(out) || (residual && !aligned16(residual)))
        return fail(MOE_ERR_INVALID_ARG, "%s: x/out NULL or rows not 16-byte aligned", who);
    return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_experts_decode(const moe_experts* routed, const moe_experts* shared,
                              const uint16_t* x, int32_t T, int32_t k, const int32_t* ids,
                              const float* weights, const uint16_t* residual, uint16_t* out,
                              void* ws, size_t ws_bytes, void* stream) {
    const moe_status st = check_decode(routed, shared, T, k, x, residual, out,
                                       "moe_experts_decode");
    if (st != MOE_OK) return st;
    if (T == 0) return ok();
    if (!ids || !weights)
        return fail(MOE_ERR_INVALID_ARG, "moe_experts_decode: ids/weights NULL");
    const size_t need = moe::decode_ws_layout(T, k, routed->d_model, routed->d_ff).bytes;
    if (!ws || ws_bytes < need || !aligned16(ws))
        return fail(MOE_ERR_WORKSPACE, "moe_experts_decode: needs %zu workspace bytes (got %zu)",
                    need, ws_bytes);
    // no logits: the kernels only read ids and weights
    return hip_status(moe::launch_decode_ffn(*routed, shared, x, T, k, nullptr,
                                             const_cast<int32_t*>(ids),
                                             const_cast<float*>(weights), residual, nullptr,
                                             out, ws,
                                             static_cast<hipStream_t>(stream)),
                      "moe_experts_decode");
}

}  // extern "C"

namespace {

// Argument checks of moe_layer_decode and moe_layer_decode_noalloc; *need = workspace bytes.
moe_status check_layer_decode(const moe_router* r, const moe_experts* routed,
                              const moe_experts* shared, const uint16_t* x, int32_t T,
                              int32_t k, int32_t* ids, float* weights,
                              const uint16_t* residual, uint16_t* out, const char* who,
                              size_t* need) {
    moe_status st = check_router(r, who);
    if (st != MOE_OK) return st;
    st = check_decode(routed, shared, T, k, x, residual, out, who);
    if (st != MOE_OK) return st;
    const int E = r->n_experts, d = r->d_model, F = routed->d_ff;
    if (routed->n_experts != E || routed->d_model != d)
        return fail(MOE_ERR_INVALID_ARG,
                    "%s: router (E %d, d %d) and experts (E %d, d %d) differ", who, E, d,
                    routed->n_experts, routed->d_model);
    *need = T > 0 ? decode_ws(T, k, E, d, F) : 0;
    if (T > 0 && (!ids || !weights)) return fail(MOE_ERR_INVALID_ARG, "%s: ids/weights NULL", who);
    return MOE_OK;
}

// The three launches of the decode layer on a workspace of decode_ws bytes.
moe_status run_layer_decode(const moe_router* r, const moe_experts* routed,
                            const moe_experts* shared, const uint16_t* x, int32_t T, int32_t k,
                            int32_t* ids, float* weights, const uint16_t* residual,
                            uint16_t* out, void* ws, hipStream_t s) {
    const int E = r->n_experts;
    uint8_t* base = static_cast<uint8_t*>(ws);
    unsigned* counter = reinterpret_cast<unsigned*>(base);
    float* lg = reinterpret_cast<float*>(base + moe::kRouteCounterBytes);
    uint8_t* ffn_ws = base + round_up(route_exact_ws(T, E));
    hipError_t e;
    if (T <= moe::kDecodeSelectMaxTokens) {
        // logits only; every gate/up block selects its token's experts itself
        e = moe::launch_route_logits(*r, x, T, lg, s);
        if (e != hipSuccess) return hip_status(e, "moe_layer_decode: route");
        e = moe::launch_decode_ffn(*routed, shared, x, T, k, lg, ids, weights, residual,
                                   nullptr, out, ffn_ws, s);
    } else {
        // several tokens: the route kernel selects once (its last block, one wave per
        // token) instead of every gate/up block repeating one token's selection
        e = moe::launch_route(*r, x, T, k, ids, weights, lg, counter, s);
        if (e != hipSuccess) return hip_status(e, "moe_layer_decode: route");
        e = moe::launch_decode_ffn(*routed, shared, x, T, k, nullptr, ids, weights, residual,
                                   nullptr, out, ffn_ws, s);
    }
    return hip_status(e, "moe_layer_decode");
}

}  // namespace

extern "C" {

moe_status moe_layer_decode(const moe_router* r, const moe_experts* routed,
                            const moe_experts* shared, const uint16_t* x, int32_t T, int32_t k,
                            int32_t* ids, float* weights, const uint16_t* residual,
                            uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
    size_t need = 0;
    const moe_status st = check_layer_decode(r, routed, shared, x, T, k, ids, weights,
                                             residual, out, "moe_layer_decode", &need);
    if (st != MOE_OK) return st;
    if (T == 0) return ok();
    if (!ws || ws_bytes < need || !aligned16(ws))
        return fail(MOE_ERR_WORKSPACE, "moe_layer_decode: needs %zu workspace bytes (got %zu)",
                    need, ws_bytes);
    return run_layer_decode(r, routed, shared, x, T, k, ids, weights, residual, out, ws,
                            static_cast<hipStream_t>(stream));
}

// ---- moe_layer_decode_noalloc: the workspace is the file-scope array `scratch`
}  // extern "C"

namespace {

__global__ void zero_words_kernel(unsigned* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_base[kMaxDevices] = {};

// Device address of this GPU's `scratch`, looked up once per device with that device
// current.  The first call on a device also clears the route counter area (the only part
// that must start at zero; every call leaves it zero again) with a fill kernel on `s`.
hipError_t scratch_base(hipStream_t s, void** base) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_base[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        constexpr int n = (int)(moe::kRouteCounterBytes / sizeof(unsigned));
        zero_words_kernel<<<1, n, 0, s>>>(static_cast<unsigned*>(p), n);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        g_scratch_base[dev] = p;
    }
    *base = g_scratch_base[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

moe_status moe_layer_decode_noalloc(const moe_router* r, const moe_experts* routed,
                                    const moe_experts* shared, const uint16_t* x, int32_t T,
                                    int32_t k, int32_t* ids, float* weights,
                                    const uint16_t* residual, uint16_t* out, void* stream) {
    size_t need = 0;
    const moe_status st = check_layer_decode(r, routed, shared, x, T, k, ids, weights,
                                             residual, out, "moe_layer_decode_noalloc", &need);
    if (st != MOE_OK) return st;
    if (T == 0) return ok();
    if (need > kNoAllocScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED,
                    "moe_layer_decode_noalloc: this call needs %zu workspace bytes, more than "
                    "the %zu of the library's fixed workspace; use moe_layer_decode", need,
                    kNoAllocScratchBytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void* base = nullptr;
    const hipError_t e = scratch_base(s, &base);
    if (e != hipSuccess) return hip_status(e, "moe_layer_decode_noalloc: fixed workspace");
    return run_layer_decode(r, routed, shared, x, T, k, ids, weights, residual, out, base, s);
}

moe_status moe_rmsnorm(const moe_norm* n, const uint16_t* x, int32_t T, int32_t d,
                       uint16_t* xn, float* z, void* stream) {
    const moe_status st = check_norm(n, d, "moe_rmsnorm");
    if (st != MOE_OK) return st;
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_rmsnorm: T = %d < 0", T);
    if (T == 0) return ok();
    if (!x || !aligned16(x) || !xn || !aligned16(xn))
        return fail(MOE_ERR_INVALID_ARG, "moe_rmsnorm: x/xn NULL or not 16-byte aligned");
    if (n->gate_w && !z)
        return fail(MOE_ERR_INVALID_ARG, "moe_rmsnorm: a gate row needs z");
    return hip_status(moe::launch_rmsnorm(x, T, d, n->gamma, n->eps, n->gate_w, n->gate_b, xn,
                                          n->gate_w ? z : nullptr,
                                          static_cast<hipStream_t>(stream)),
                      "moe_rmsnorm");
}

moe_status moe_combine_gated(const uint16_t* y_pairs, const int32_t* pair_pos,
                             const float* weights, const uint16_t* y_shared, const float* z,
                             const uint16_t* residual, int32_t T, int32_t k, int32_t d,
                             uint16_t* out, void* stream) {
    if (T > 0 && !z) return fail(MOE_ERR_INVALID_ARG, "moe_combine_gated: z NULL");
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "moe_combine_gated: T = %d < 0", T);
    if (k < 1 || k > kMaxK) return fail(MOE_ERR_INVALID_ARG, "moe_combine_gated: k = %d", k);
    if (d < 8 || d % 8 != 0) return fail(MOE_ERR_INVALID_ARG, "moe_combine_gated: d = %d", d);
    if (T == 0) return ok();
    if (!y_pairs || !pair_pos || !weights || !out)
        return fail(MOE_ERR_INVALID_ARG,
                    "moe_combine_gated: y_pairs/pair_pos/weights/out NULL");
    if (!aligned16(y_pairs) || !aligned16(out) || (y_shared && !aligned16(y_shared)) ||
        (residual && !aligned16(residual)))
        return fail(MOE_ERR_INVALID_ARG, "moe_combine_gated: bf16 rows must be 16-byte aligned");
    return hip_status(moe::launch_combine(y_pairs, pair_pos, weights, y_shared, residual, z, T,
                                          k, d, out, static_cast<hipStream_t>(stream)),
                      "moe_combine_gated");
}

moe_status moe_block_decode(const moe_norm* n, const moe_router* r, const moe_experts* routed,
                            const moe_experts* shared, const uint16_t* x, int32_t T, int32_t k,
                            int32_t* ids, float* weights, uint16_t* out, void* ws,
                            size_t ws_bytes, void* stream) {
    size_t need = 0;
    moe_status st = check_layer_decode(r, routed, shared, x, T, k, ids, weights, nullptr, out,
                                       "moe_block_decode", &need);
    if (st != MOE_OK) return st;
    st = check_norm(n, r->d_model, "moe_block_decode");
    if (st != MOE_OK) return st;
    if (T == 0) return ok();
    if (T > moe::kRouteGemvMaxTokens)
        return fail(MOE_ERR_UNSUPPORTED,
                    "moe_block_decode: T = %d above %d; use moe_rmsnorm and the four calls", T,
                    moe::kRouteGemvMaxTokens);
    const int E = r->n_experts, d = r->d_model, F = routed->d_ff;
    need = block_ws(T, k, E, d, F);
    if (!ws || ws_bytes < need || !aligned16(ws))
        return fail(MOE_ERR_WORKSPACE, "moe_block_decode: needs %zu workspace bytes (got %zu)",
                    need, ws_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* base = static_cast<uint8_t*>(ws);
    unsigned* counter = reinterpret_cast<unsigned*>(base);
    float* lg = reinterpret_cast<float*>(base + moe::kRouteCounterBytes);
    uint8_t* ffn_ws = base + round_up(route_exact_ws(T, E));
    uint16_t* xn = reinterpret_cast<uint16_t*>(base + decode_ws(T, k, E, d, F));
    float* z = n->gate_w ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(xn) +
                                                    round_up((size_t)T * d * 2))
                         : nullptr;
    // the router on xn = RMSNorm(x) (it writes xn and z); up to kDecodeSelectMaxTokens
    // tokens logits only, every gate/up block selects; more: the route kernel's last block
    // selects
    hipError_t e = moe::launch_route_norm(*r, x, T, k, n->gamma, n->eps, n->gate_w, n->gate_b,
                                          xn, z, ids, weights, lg, counter, s);
    if (e != hipSuccess) return hip_status(e, "moe_block_decode: route");
    e = moe::launch_decode_ffn(*routed, shared, xn, T, k,
                               T <= moe::kDecodeSelectMaxTokens ? lg : nullptr, ids, weights,
                               x, z, out, ffn_ws, s);
    return hip_status(e, "moe_block_decode");
}

moe_status moe_dequant_probe(int32_t fmt, int32_t form, const uint8_t* w, const uint16_t* s,
                             int64_t n_groups, void* out, void* stream) {
    if (!expert_fmt(fmt))
        return fail(MOE_ERR_INVALID_ARG,
                    "moe_dequant_probe: format %d is not INT4_G32/INT6_G32/INT3_G32/INT2_G32",
                    fmt);
    if (form != 0 && form != 1)
        return fail(MOE_ERR_INVALID_ARG, "moe_dequant_probe: form %d is not 0 or 1", form);
    if (n_groups < 0 || n_groups > ((int64_t)1 << 31))
        return fail(MOE_ERR_INVALID_ARG, "moe_dequant_probe: n_groups = %lld",
                    (long long)n_groups);
    if (n_groups == 0) return ok();
    if (!w || !s || !out || !aligned16(w) || !aligned16(out) || ((uintptr_t)s & 1u))
        return fail(MOE_ERR_INVALID_ARG,
                    "moe_dequant_probe: w/out NULL or not 16-byte aligned, or s NULL/odd");
    return hip_status(moe::launch_dequant_probe(fmt, form, w, s, n_groups, out,
                                                static_cast<hipStream_t>(stream)),
                      "moe_dequant_probe");
}

moe_status moe_check_device_error(void* stream) {
    hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_status(e, "moe_check_device_error: sync");
    int flag = 0;
    e = moe::read_and_clear_device_error(&flag);
    if (e != hipSuccess) return hip_status(e, "moe_check_device_error: read flag");
    if (flag & 1) return fail(MOE_ERR_DEVICE, "an expert id outside [0, E) was seen");
    if (flag) return fail(MOE_ERR_DEVICE, "device error flag 0x%x", flag);
    return ok();
}

}  // extern "C"
