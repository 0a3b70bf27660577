/*
 * moe.h -- C ABI of the MI355X (gfx950) quantized routed-expert MoE layer.
 *
 * The layer, as the pages describe it: each layer owns 512 routed experts, every token
 * is sent to 10 of them and to one shared expert that is always on
 * [Strata 与 Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会]; a router that
 * lives on the GPU makes the choice [本地部署Qwen3.8-Flash-Next模型的两条路线
 * (blog.cycleuser.org), section 硬件形态决定了各自的走法]; expert weights are 4-bit,
 * some mixed layers 6-bit and a dense projection 8-bit [same page, section 精度和内存占用];
 * prefill batches many tokens per expert while decode is latency bound [telli.sh page,
 * section GPU、RAM 和 SSD 各司其职].  One layer is the composition
 *
 *     moe_route -> moe_permute -> moe_expert_ffn (routed; and shared, dense) -> moe_combine
 *
 * and, for a few tokens, moe_layer_decode runs that composition in three launches on one
 * stream.
 *
 * Conventions for every entry point
 *   - Pointers to tensors are DEVICE pointers (hipMalloc'd or torch-owned memory); the
 *     descriptor structs themselves are read on the host during the call.  The caller
 *     owns all memory; the library never allocates or frees device memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *     entry point only enqueues work on that stream and returns; nothing synchronises
 *     except moe_check_device_error.
 *   - bf16 and fp16 values travel as uint16_t bit patterns.
 *   - Validation happens on the host before any launch.  A failing call launches
 *     nothing and returns a negative status; moe_last_error() has the detail (per
 *     thread).  T = 0 is a valid no-op.
 *   - Results are deterministic: the same inputs give the same bits on every run.
 *   - Workspaces: size them with moe_workspace_size and ZERO-FILL them once before their
 *     first use.  The first bytes of the route workspace hold an arrival counter that
 *     the kernel counts up and resets before it finishes, so every call leaves it zero
 *     again.  Two calls that run at the same time need two workspaces.
 *
 * Weight formats (groups of 32 consecutive elements along a row's input dimension):
 *   MOE_FMT_INT4_G32  row of K codes = K/2 bytes; byte i: element 2i in the low nibble,
 *                     2i+1 in the high nibble; value = s * (nibble - 8); one fp16 scale
 *                     s per group, scales [rows][K/32].
 *   MOE_FMT_INT6_G32  row = K*3/4 bytes; each group of 32 codes is a 24-byte
 *                     little-endian bit string, code i at bits [6i, 6i+6);
 *                     value = s * (code - 32).
 *   MOE_FMT_INT3_G32  row = K*3/8 bytes; a group is a 12-byte little-endian bit string,
 *                     code i at bits [3i, 3i+3); value = s * (code - 4).
 *   MOE_FMT_INT2_G32  row = K/4 bytes; a group is 8 bytes, code i at bits [2i, 2i+2);
 *                     value = s * (code - 2).
 *   (int3 and int2 are this library's own plain codecs for the low-bit expert tiers of
 *   [Strata 与 Qwen3.8-Flash-Next (telli.sh)]: not the GGUF formats those tiers use.)
 *   MOE_FMT_INT8_ROW  router only: int8 [E][d] with one fp16 scale per row.
 *   MOE_FMT_FP32      router only: fp32 [E][d].
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1,   /* null pointer, bad size, misalignment, bad format */
    MOE_ERR_UNSUPPORTED = -2,   /* valid request this library has no kernel for */
    MOE_ERR_WORKSPACE = -3,     /* workspace missing or smaller than moe_workspace_size */
    MOE_ERR_HIP = -4,           /* a HIP runtime call failed (launch, sync, copy) */
    MOE_ERR_DEVICE = -5         /* a kernel reported bad data (expert id out of range) */
};

enum {
    MOE_FMT_FP32 = 0,
    MOE_FMT_INT8_ROW = 1,
    MOE_FMT_INT4_G32 = 2,
    MOE_FMT_INT6_G32 = 3,
    MOE_FMT_INT3_G32 = 4,
    MOE_FMT_INT2_G32 = 5
};

/* Operation ids for moe_workspace_size. */
enum {
    MOE_OP_ROUTE = 0,
    MOE_OP_PERMUTE = 1,
    MOE_OP_EXPERT_FFN = 2,
    MOE_OP_LAYER_DECODE = 3,
    MOE_OP_EXPERTS_DECODE = 4,
    MOE_OP_BLOCK_DECODE = 5
};

/* Router: logits = W x (+ bias).  fmt FP32: w = fp32 [E][d], scale unused.
 * fmt INT8_ROW: w = int8 [E][d], scale = fp16 [E].  bias = fp32 [E] or NULL.
 * Needs d % 256 == 0 (FP32) or d % 1024 == 0 (INT8_ROW); 1 <= E <= 1024. */
typedef struct moe_router {
    int32_t fmt;
    int32_t n_experts;
    int32_t d_model;
    int32_t reserved;        /* must be 0 */
    const void* w;
    const uint16_t* scale;
    const float* bias;
} moe_router;

/* A set of E experts of one format (INT4_G32, INT6_G32, INT3_G32 or INT2_G32).  Expert e:
 *   gate, up : [d_ff][d_model] -> w_gate/w_up bytes [E][d_ff][row bytes(d_model)],
 *              s_gate/s_up fp16 [E][d_ff][d_model/32]
 *   down     : [d_model][d_ff] -> w_down bytes [E][d_model][row bytes(d_ff)],
 *              s_down fp16 [E][d_model][d_ff/32]
 * The shared expert is a set with E = 1.  d_model must be one of 256, 512, 1024, 2048,
 * 4096 and d_ff one of 128, 256, ..., 4096; weight and scale pointers must be 16-byte
 * aligned. */
typedef struct moe_experts {
    int32_t fmt;
    int32_t n_experts;
    int32_t d_model;
    int32_t d_ff;
    const uint8_t* w_gate;
    const uint8_t* w_up;
    const uint8_t* w_down;
    const uint16_t* s_gate;
    const uint16_t* s_up;
    const uint16_t* s_down;
} moe_experts;

/* The pre-layer RMS norm and the residual gate of a MoE block (moe_rmsnorm,
 * moe_combine_gated, moe_block_decode).  The pages keep a gated residual on the GPU next to
 * the router and the shared expert [本地部署Qwen3.8-Flash-Next模型的两条路线
 * (blog.cycleuser.org), section 硬件形态决定了各自的走法] without a formula; the reading
 * here: the layer runs on xn = RMSNorm(x) and its output joins the residual stream as
 * x_next = bf16(x + bf16(sigmoid(z) * out)), z = <gate_w, xn> + gate_b per token.
 *   gamma   fp32 [d] per-channel scale of the norm (16-byte aligned)
 *   gate_w  fp32 [d] residual-gate row (16-byte aligned), or NULL: no gate (factor 1)
 *   eps     added to the mean square (finite, >= 0)
 *   gate_b  residual-gate bias (finite) */
typedef struct moe_norm {
    const float* gamma;
    const float* gate_w;
    float eps;
    float gate_b;
} moe_norm;

/*
 * moe_rmsnorm -- xn = RMSNorm(x) for T tokens, and their residual-gate logits.
 *   x   bf16 [T][d]; xn bf16 [T][d] out; z fp32 [T] out (needed when gate_w != NULL,
 *       ignored otherwise).  d = 256, 512, 1024, 2048 or 4096.
 * Fixed fp32 arithmetic, so that routing on xn is reproducible bit for bit: ss = sum of
 * x_c^2 with the row cut into chunks of 4 elements, chunk v to lane v mod 64, one fused
 * multiply-add chain per lane over its chunks in ascending order, then a butterfly over the
 * 64 lanes with offsets 1..32; r = fl(1 / fl(sqrt(fl(fl(ss / d) + eps)))) with IEEE
 * division and square root; xn_c = bf16(fl(fl(x_c * r) * gamma_c)).  z = <gate_w, xn> +
 * gate_b in moe_route's fixed fp32 order.  One launch.
 */
moe_status moe_rmsnorm(const moe_norm* n, const uint16_t* x, int32_t T, int32_t d,
                       uint16_t* xn, float* z, void* stream);

/*
 * moe_route -- router logits, top-k selection and gate weights for T tokens.  A router
 * picks 10 of each layer's 512 routed experts for every token [Strata 与 Qwen3.8-Flash-Next
 * (telli.sh), section 稀疏架构创造了机会] and stays on the GPU [本地部署Qwen3.8-Flash-Next
 * 模型的两条路线 (blog.cycleuser.org), section 硬件形态决定了各自的走法]; the linear map, the
 * summation order and the softmax over the selected logits are this library's readings.
 *   x       bf16 [T][d] (16-byte aligned)
 *   ids     int32 [T][k]: out; the k experts with the largest fp32 logits, slot 0 the
 *           largest; equal logits (+0 == -0) -> lower expert id first
 *   weights fp32 [T][k]: out; softmax over the k selected logits (the full softmax
 *           renormalised over the selected experts); sums to 1 up to rounding
 *   logits  fp32 [T][E]: optional out (NULL: not returned; see below)
 *   ws      zero-initialised workspace of moe_workspace_size(MOE_OP_ROUTE, T, k, E, d, 0)
 *           bytes (256 bytes are enough when logits != NULL)
 * Logits are defined in one fixed fp32 order, the same for every T: the row is cut into
 * 16-byte vectors dealt round-robin to 64 lanes, each lane runs one fused-multiply-add
 * chain over its vectors in ascending order, and the 64 lane sums are combined by a
 * butterfly with offsets 1, 2, 4, ..., 32; then + bias (FP32), or
 * fl(fl(sum * scale) + bias) (INT8_ROW).  ids and weights are always those of these
 * logits.  How they are reached:
 *   T <= 4: logits and selection in one launch (the last block to finish its rows
 *            selects);
 *   4 < T <= 512: the same one-wave-per-expert-row logits (eight tokens and up to two
 *            rows per wave), then a selection kernel (a wave per token);
 *   T > 512, logits requested: an LDS-tiled fp32 GEMM in the fixed order, then selection;
 *   T > 512, logits NULL (the bounded form): bf16 MFMA logits (FP32 rows split exactly
 *            into two bf16 parts plus a dropped remainder below 2^-17 of the weight)
 *            within 2^-11 (|x_t| |w_e| + |b_e|) of the fixed-order value; per token the
 *            experts that this bound cannot rule out of the top k are recomputed in the
 *            fixed order, and the selection runs over exact values for them.  The ids and
 *            weights are bit for bit those of the other forms.  Three launches; the
 *            workspace then also holds the logits, bf16 copies of the router rows and
 *            their norms (moe_workspace_size accounts for them).
 * Requires 1 <= k <= min(E, 64).
 */
moe_status moe_route(const moe_router* r, const uint16_t* x, int32_t T, int32_t k,
                     int32_t* ids, float* weights, float* logits, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * moe_permute -- group the P = T*k (token, slot) pairs by expert, stably.  Prefill runs
 * many tokens through each expert in one batch [Strata 与 Qwen3.8-Flash-Next (telli.sh),
 * section GPU、RAM 和 SSD 各司其职], which needs each expert's pairs contiguous.
 *   ids           int32 [T][k] expert ids from moe_route
 *   offsets       int32 [E+1]: out; expert e's pairs are sorted_pairs[offsets[e] ..
 *                 offsets[e+1]); offsets[E] = number of valid pairs
 *   sorted_pairs  int32 [P]: out; pair indices p = t*k + j, by expert then by p
 *   pair_pos      int32 [P]: out; position of pair p in sorted_pairs (-1 if its id is
 *                 outside [0, E): such pairs are dropped and the device error flag read
 *                 by moe_check_device_error is raised)
 *   ws            moe_workspace_size(MOE_OP_PERMUTE, T, k, E, 0, 0) bytes
 * Integer-exact; no order-dependent atomics.
 */
moe_status moe_permute(const int32_t* ids, int32_t T, int32_t k, int32_t E,
                       int32_t* offsets, int32_t* sorted_pairs, int32_t* pair_pos,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_ffn -- y = Wd (silu(Wg x) * (Wu x)) for every (token, expert) pair: the
 * routed experts a token activates and the always-on shared expert [Strata 与
 * Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会], their weights stored at 4 bit
 * (6 bit in mixed layers) [本地部署Qwen3.8-Flash-Next模型的两条路线 (blog.cycleuser.org),
 * section 精度和内存占用] or 2-3 bit in low-bit tiers [Strata 与 Qwen3.8-Flash-Next
 * (telli.sh)]; decode reads the active experts' weights once per step [Halogen Flash
 * Server配置與實測 (lcz.me), replies comparing decode with bandwidth].
 * Grouped mode (routed experts): ids, offsets, sorted_pairs from moe_route/moe_permute;
 *   y is bf16 [T*k][d] in sorted order: row i belongs to pair sorted_pairs[i] and its
 *   token sorted_pairs[i] / k.  Rows past offsets[E] are left untouched.
 * Dense mode (shared expert): ids, offsets and sorted_pairs all NULL, ex->n_experts == 1,
 *   k ignored; y is bf16 [T][d], row t for token t.
 * Arithmetic: fp32 accumulation of bf16 activations times dequantised weights; the
 * hidden activation h = silu(g) * u is rounded to bf16 before the down projection.
 * Decode-sized calls on a (d_model, d_ff) pair with a GEMV kernel ((2048, 512),
 * (2048, 1024), (2048, 2048), (4096, 1024), (1024, 512), (256, 128)) stream each selected
 * expert's weights (two launches: gate/up + SwiGLU, then down):
 *   at most 24 pairs (grouped), or at most 64 rows (dense): each pair's row is derived
 *     from ids alone (dense: the token index); offsets and sorted_pairs
 *     are not read, so moe_permute may run concurrently with the call;
 *   more than 24 pairs (grouped mode): a third, earlier launch lists each expert's sorted
 *     positions in chunks of at most 3 from offsets and sorted_pairs (so moe_permute must
 *     have completed), and each chunk streams its expert's weights once; from 640 rows an
 *     expert with 8 or more pairs (4 or more above 1024 rows) runs the grouped MFMA GEMM
 *     below instead, in two more launches on the same h and y.
 * A pair's output bits are the same whenever it runs on the GEMV (and the same in
 * moe_layer_decode); on the GEMM they differ by rounding.  Dense calls above 64 tokens, and
 * shapes without a GEMV kernel, run the grouped MFMA GEMM alone, reading offsets and
 * sorted_pairs.  Wherever the GEMM may run it needs T*d_model and T*k*d_ff (dense: T*d_ff)
 * below 2^31 elements (MOE_ERR_UNSUPPORTED otherwise: split the call).
 * ws: moe_workspace_size(MOE_OP_EXPERT_FFN, T, k, E, d, d_ff) bytes (pass k = 1, E = 1
 * for dense mode).
 */
moe_status moe_expert_ffn(const moe_experts* ex, const uint16_t* x, int32_t T, int32_t k,
                          const int32_t* ids, const int32_t* offsets,
                          const int32_t* sorted_pairs, uint16_t* y, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * moe_combine -- out[t] = bf16( sum_{j<k} w[t][j] * y_pairs[pair_pos[t*k+j]]  + y_shared[t] )
 * with the sum taken in fp32 over slots j = 0..k-1 in order, then the shared row added,
 * then one rounding to bf16.  y_shared may be NULL.  Pairs with pair_pos < 0 contribute
 * nothing.  If residual (bf16 [T][d]) is not NULL the stored value is instead
 * bf16(residual + bf16(that sum)), the next layer's input in a stacked sweep.
 * out may alias residual.  Needs d % 8 == 0 and 16-byte aligned rows.
 * A token's output is its selected experts weighted by the router plus the shared expert
 * [Strata 与 Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会]; the slot order and
 * the single rounding are this library's readings.
 */
moe_status moe_combine(const uint16_t* y_pairs, const int32_t* pair_pos, const float* weights,
                       const uint16_t* y_shared, const uint16_t* residual, int32_t T,
                       int32_t k, int32_t d, uint16_t* out, void* stream);

/*
 * moe_combine_gated -- moe_combine with the residual gate: the fp32 sum of moe_combine
 * (slots in order, then the shared row) is scaled once by g = sigmoid(z[t]) =
 * 1 / (1 + exp(-z[t])) before its rounding: out = bf16(residual + bf16(fl(g * sum))), or
 * bf16(fl(g * sum)) without a residual.  z fp32 [T] (required); other arguments as in
 * moe_combine.
 */
moe_status moe_combine_gated(const uint16_t* y_pairs, const int32_t* pair_pos,
                             const float* weights, const uint16_t* y_shared, const float* z,
                             const uint16_t* residual, int32_t T, int32_t k, int32_t d,
                             uint16_t* out, void* stream);

/*
 * moe_layer_decode -- the whole layer for a few tokens (decode, MTP verification): the same
 * result, bit for bit, as
 *     moe_route -> moe_permute -> moe_expert_ffn(routed) -> moe_expert_ffn(shared, dense)
 *     -> moe_combine(residual)
 * on the same inputs, in three launches on `stream`.  One token: the router GEMV (logits
 * only), a gate/up kernel whose blocks each select the token's experts (and write ids and
 * weights), then a down kernel that produces a few output rows of every pair per block and
 * combines them in registers (y never goes to memory).  Several tokens: moe_route's kernel
 * (logits and selection), then the same gate/up kernel with the ids given, then the same
 * down kernel.  Each token is sent to k experts and to the shared one, as the layer the pages
 * describe [Strata 与 Qwen3.8-Flash-Next (telli.sh), section 稀疏架构创造了机会].
 *   routed   the routed expert set; n_experts and d_model must match the router's
 *   shared   the shared expert (n_experts 1, same format, d_model and d_ff) or NULL
 *   x        bf16 [T][d]; ids int32 [T][k] and weights fp32 [T][k] are outputs as in
 *            moe_route; residual bf16 [T][d] or NULL; out bf16 [T][d] (may alias residual)
 *   ws       zero-initialised workspace of moe_workspace_size(MOE_OP_LAYER_DECODE, T, k,
 *            E, d, d_ff) bytes; its first bytes hold moe_route's arrival counter, which
 *            every call leaves zero again
 * Needs T*k <= 64, the h rows of all T*k (+ T shared) slots within 128 KiB of LDS, and a
 * (d_model, d_ff) pair with a GEMV kernel (see moe_expert_ffn); otherwise
 * MOE_ERR_UNSUPPORTED and the caller uses the four calls.
 */
moe_status moe_layer_decode(const moe_router* r, const moe_experts* routed,
                            const moe_experts* shared, const uint16_t* x, int32_t T, int32_t k,
                            int32_t* ids, float* weights, const uint16_t* residual,
                            uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_block_decode -- one MoE block of a stacked model for a few tokens: the pre-layer norm,
 * the layer, and the gated residual, fused into moe_layer_decode's three launches (the norm
 * inside the router kernel, the gate inside the down kernel's combine).  The result equals,
 * bit for bit,
 *     moe_rmsnorm -> moe_route(xn) -> moe_permute -> moe_expert_ffn(routed, xn)
 *     -> moe_expert_ffn(shared, dense, xn) -> moe_combine_gated(z, residual = x)
 * (without a gate row: moe_combine with residual = x).  48 such blocks are stacked in the
 * model the pages describe [Strata 与 Qwen3.8-Flash-Next (telli.sh), section
 * 稀疏架构创造了机会].
 *   n        the block's norm and residual gate; r, routed, shared as in moe_layer_decode
 *   x        bf16 [T][d], the block's input (the residual stream)
 *   ids, weights  out, as in moe_route (of xn)
 *   out      bf16 [T][d]: x_next; may alias x
 *   ws       zero-initialised workspace of moe_workspace_size(MOE_OP_BLOCK_DECODE, T, k, E,
 *            d, d_ff) bytes (it holds xn and z too); its counter is left zero by every call
 * Needs what moe_layer_decode needs and T <= 16 (MOE_ERR_UNSUPPORTED otherwise).
 */
moe_status moe_block_decode(const moe_norm* n, const moe_router* r, const moe_experts* routed,
                            const moe_experts* shared, const uint16_t* x, int32_t T, int32_t k,
                            int32_t* ids, float* weights, uint16_t* out, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * moe_layer_decode_noalloc -- moe_layer_decode for callers that cannot allocate device
 * memory or pass a workspace: code recorded under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, checks and results (bit for bit) as
 * moe_layer_decode, without ws / ws_bytes: the workspace is a fixed 512 KiB array inside
 * the library, one per GPU, held until the process ends.  Every valid decode call fits
 * (moe_workspace_size(MOE_OP_LAYER_DECODE, ...) is at most 472.25 KiB over every shape
 * moe_layer_decode accepts); a larger need would return MOE_ERR_UNSUPPORTED.  The call allocates nothing.  Its first call on a GPU looks
 * up that GPU's array and enqueues one small kernel on `stream` that clears its counter
 * area.  All calls on one GPU share the array, so two calls whose work overlaps on the
 * GPU (different streams, no ordering between them) race and give undefined results;
 * calls ordered on one stream are safe.
 */
moe_status moe_layer_decode_noalloc(const moe_router* r, const moe_experts* routed,
                                    const moe_experts* shared, const uint16_t* x, int32_t T,
                                    int32_t k, int32_t* ids, float* weights,
                                    const uint16_t* residual, uint16_t* out, void* stream);

/*
 * moe_experts_decode -- the last two launches of moe_layer_decode on their own: given ids
 * and weights from moe_route, the routed and shared expert FFNs and the combine, bit for
 * bit equal to moe_permute -> moe_expert_ffn x 2 -> moe_combine.  Arguments as in
 * moe_layer_decode; ws: moe_workspace_size(MOE_OP_EXPERTS_DECODE, T, k, E, d, d_ff) bytes
 * (no zero-fill needed).  An id outside [0, n_experts) (moe_route never gives one) reads
 * expert 0 and raises the device error flag (moe_check_device_error).
 */
moe_status moe_experts_decode(const moe_experts* routed, const moe_experts* shared,
                              const uint16_t* x, int32_t T, int32_t k, const int32_t* ids,
                              const float* weights, const uint16_t* residual, uint16_t* out,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * moe_dequant_probe -- a verification entry point: runs the weight decoder of one of the
 * two expert paths over n_groups consecutive 32-code groups of a packed matrix, so that
 * every decoded weight can be compared bit for bit with its exact value s * q (expert
 * weights at 4 and 6 bit [本地部署Qwen3.8-Flash-Next模型的两条路线 (blog.cycleuser.org),
 * section 精度和内存占用]).
 *   fmt   MOE_FMT_INT4_G32, MOE_FMT_INT6_G32, MOE_FMT_INT3_G32 or MOE_FMT_INT2_G32
 *   w     packed codes of n_groups groups (16, 24, 12 or 8 bytes each), device, 16-byte
 *         aligned
 *   s     fp16 scales [n_groups], device
 *   form 0: out fp32 [n_groups][32]: the few-token (GEMV) kernels' group arithmetic
 *           (dot product on offset codes, zero-point removal, scale) evaluated on one-hot
 *           activations; equals s * q exactly when the decoder is right.
 *   form 1: out bf16 [n_groups][32]: the grouped GEMM's MFMA operand, bf16(s * q) rounded
 *           to nearest even.
 * Enqueues one launch on `stream`.  n_groups = 0 is a no-op; above 2^31 is rejected.
 */
moe_status moe_dequant_probe(int32_t fmt, int32_t form, const uint8_t* w, const uint16_t* s,
                             int64_t n_groups, void* out, void* stream);

/* Workspace bytes an operation needs for these sizes (0 = none).  0 also for sizes that
 * every call of the operation rejects: T, k or n_experts not positive, more than 1024
 * experts, more than 2^31 - 1 (token, expert) pairs, or (MOE_OP_ROUTE above 512 tokens) a
 * d_model that is not positive.  For the decode operations (MOE_OP_LAYER_DECODE,
 * MOE_OP_EXPERTS_DECODE, MOE_OP_BLOCK_DECODE) 0 also means that they do not run for these
 * sizes (more than 64 pairs, or a (d_model, d_ff) pair without decode kernels): the call
 * returns MOE_ERR_UNSUPPORTED.  Pure host function. */
size_t moe_workspace_size(int32_t op, int32_t T, int32_t k, int32_t E, int32_t d,
                          int32_t d_ff);

/* Synchronises `stream`, then reports and clears the current device's error flag:
 * MOE_ERR_DEVICE if, since the last check, a kernel saw an expert id outside [0, E). */
moe_status moe_check_device_error(void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status s);

/* Detail of the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

/* Library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
