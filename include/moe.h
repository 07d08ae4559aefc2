/*
 * moe.h - C ABI of the MI355X (gfx950) routed int4 Mixture-of-Experts layer.
 *
 * The layer is the routed-expert block of Qwen3.6-35B-A3B: E routed experts,
 * top-k routing plus one shared expert, SwiGLU experts whose gate, up and down
 * projections are affine 4-bit in groups of 64, and an 8-bit (or fp32) router.
 * Sources (the pages are cited by title and section):
 *   [P3-build] TensorFold issue #931, "Qwen3.6-35B-A3B (qwen3_5_moe) on the native
 *              Metal engine: proposal and gate", section "What I'd build": the routing
 *              contract (fp32 logits over the experts and the shared gate; top-k by
 *              logit, ties to the lower id; weights exp(l - l_top) over the k picks
 *              rounded to bf16; the shared expert as one more slot weighted
 *              bf16(sigmoid(bf16(gate))); the weighted sum rounded once to bf16),
 *              affine 4-bit experts in groups of 64, 8-bit routers, and the refusal
 *              of other bit widths; "windows of 1 to 16 rows" for decode.
 *   [P3-what]  same page, section "What it is": routed experts replace the dense MLP;
 *              256 experts, 8 picked per token, one shared expert.
 *   [P3-gate]  same page, section "Gate": the expert gate/up pair, expert down and the
 *              combine as the projection classes of the layer.
 *   [P1-phase] "POC for qwen3.5 / qwen3.6 support optimized for AGX Orin", summary
 *              "Phase 1-4" (parallel top-k router, GEMV MoE path at batch 1) and
 *              "Phase 9b" (MoE GEMM with int4 dequant and lookup-table dispatch).
 *   [P4-run]   "Qwen-3.6-35B-A3B-SIQ-K6+K4K3", section "How to run": the shared
 *              expert gate is an N=1 projection.
 *   [P2-next]  "R9700: the 35B only one runtime could load" (R9700 vLLM blog, part 13),
 *              its closing list of kernel work: upcast the experts to FP8 to run them
 *              on the FP8 matrix units as well.
 *
 * Conventions for every call:
 *   - Pointers named *_host are host memory; every other pointer is device memory
 *     on the current HIP device, 16-byte aligned. The library never allocates or
 *     frees memory: the caller owns every buffer (inputs, outputs, workspace).
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call that
 *     launches work is asynchronous on that stream and never synchronises the host.
 *   - Arguments are validated on the host before any launch; a failed check returns
 *     MOE_ERR_INVALID_ARG / MOE_ERR_UNSUPPORTED / MOE_ERR_WORKSPACE and launches
 *     nothing. A failed launch returns MOE_ERR_HIP. moe_last_error() then holds a
 *     message (per host thread). No C++ exception crosses this boundary.
 *   - bf16 values are passed as uint16_t bit patterns.
 *   - T is the number of token rows; S = top_k + has_shared slots per token; slot
 *     s < top_k belongs to expert ids[t, s], slot top_k (if has_shared) to the
 *     shared expert. R = n_experts + has_shared router rows (row n_experts is the
 *     shared-expert gate, [P4-run]).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* bad pointer, size or shape field                */
    MOE_ERR_UNSUPPORTED = -2, /* well-formed but not served (bit width, group ...) */
    MOE_ERR_WORKSPACE = -3,   /* caller buffer smaller than the documented size   */
    MOE_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed        */
    MOE_ERR_TIMEOUT = -5      /* a bounded in-kernel wait timed out (moe_decode_layer_check) */
} moe_status;

enum { MOE_ROUTER_F32 = 0, MOE_ROUTER_AFFINE8 = 1 };

/* Layer shape and formats. Served: bits == 4 (affine 4-bit experts) or 8 (affine
 * 8-bit experts, the second checkpoint format of [P3-build]), group == 64 (any
 * other bit width or group is refused with MOE_ERR_UNSUPPORTED, as [P3-build]
 * refuses the widths a backend does not serve); hidden is a power of two in
 * [64, 8192] (8-bit: [64, 4096]), inter a power of two in [64, 2048] (8-bit:
 * [64, 1024]); 1 <= top_k <= min(n_experts, 16); 1 <= n_experts <= 1024;
 * has_shared in {0, 1}; router_fmt one of MOE_ROUTER_*. */
typedef struct moe_shape {
    int32_t hidden;     /* H: model width                          */
    int32_t inter;      /* I: expert intermediate width            */
    int32_t n_experts;  /* E: routed experts                       */
    int32_t top_k;      /* k: experts picked per token             */
    int32_t has_shared; /* 1: one shared expert (expert index E)   */
    int32_t group;      /* quantisation group along the input dim  */
    int32_t bits;       /* expert weight bits                      */
    int32_t router_fmt; /* MOE_ROUTER_F32 or MOE_ROUTER_AFFINE8    */
} moe_shape;

/* Canonical expert weights ([P3-build]: affine 4-bit, groups of 64), device memory.
 * For each of the M = n_experts + has_shared experts (index n_experts = shared):
 *   q_gate, q_up [M][I][H/2] uint8, q_down [M][H][I/2] uint8: row-major matrices
 *     [out, in] with input element 2j in the low nibble of byte j and 2j+1 in the
 *     high nibble; q in 0..15.
 *   bits == 8: q_gate, q_up [M][I][H] uint8, q_down [M][H][I] uint8, one code q in
 *     0..255 per byte.
 *   s_*, b_* [M][rows][in/64] bf16: scale and bias of each group of 64 consecutive
 *     input elements; the weight is scale * q + bias. */
typedef struct moe_expert_canon {
    const uint8_t* q_gate;
    const uint16_t* s_gate;
    const uint16_t* b_gate;
    const uint8_t* q_up;
    const uint16_t* s_up;
    const uint16_t* b_up;
    const uint8_t* q_down;
    const uint16_t* s_down;
    const uint16_t* b_down;
} moe_expert_canon;

/* ABI revision of this header. */
int32_t moe_abi_version(void);

/* Static text for a status code. */
const char* moe_status_str(int32_t status);

/* Message for the last non-OK status returned on this host thread ("" if none). */
const char* moe_last_error(void);

/* Checks a shape against the served set; MOE_OK if every call below accepts it. */
moe_status moe_shape_check(const moe_shape* shape);

/* ---------------------------------------------------------------- weight packing
 * The kernels read one packed buffer per layer. Per expert m (stride
 * moe_experts_packed_bytes / M), in this order:
 *   gate/up q [I/2][H/64][4][32 B] | down q [H/4][I/64][4][32 B] |
 *   gate/up sb [I/2][H/64][4] | down sb [H/4][I/64][4]
 * (4-bit rows; 8-bit rows are packed as 4-bit rows of twice the length: codes
 * 0 .. K-1 of an 8-bit row of K codes become the high nibbles of its codes, with
 * the group words (16 scale, bias), and codes K .. 2K-1 the low nibbles, with
 * (scale, 0): 16 s hi + b + s lo = s q + b exactly. An 8-bit expert takes twice the
 * 4-bit expert's bytes, 6 % more than its canonical 8-bit form.)
 * Rows come in blocks of four: gate/up block b holds gate rows 2b, 2b+1 and up
 * rows 2b, 2b+1 (in that slot order), down block b holds down rows 4b .. 4b+3.
 * For each block and 64-wide group g, the four rows' 32 bytes of that group
 * (their weights 64g .. 64g+63, canonical byte order) follow one another, so one
 * 128-byte line holds one group of a whole block. Every sb entry is a uint32
 * holding the group's bf16 scale in the low and bf16 bias in the high half, in
 * the same block, group, slot order. Within every little-endian dword (weights
 * k0..k7 of a row) the eight nibbles are reordered: nibble j (bits 4j..4j+3)
 * holds k_{2j} and nibble 4+j holds k_{2j+1}, j < 4. A shift by 4j then puts the
 * pair (k_{2j}, k_{2j+1}) in bits 0..3 and 16..19, i.e. next to each other as
 * they sit in a bf16 activation row. */
size_t moe_experts_packed_bytes(const moe_shape* shape);

/* Packs canonical expert weights (device) into `packed` (device, packed_bytes >=
 * moe_experts_packed_bytes). Async on `stream`. */
moe_status moe_pack_experts(const moe_shape* shape, const moe_expert_canon* src_host,
                            void* packed, size_t packed_bytes, void* stream);

/* Packed router: MOE_ROUTER_AFFINE8: q [R][H] uint8 | sb [R][H/64] uint32 (scale low,
 * bias high); MOE_ROUTER_F32: w [R][H] float. [P3-build]: routers at 8 bits. */
size_t moe_router_packed_bytes(const moe_shape* shape);

/* Packs the router. AFFINE8: w = q [R][H] uint8, s and b bf16 [R][H/64].
 * F32: w = float [R][H], s and b must be NULL. Device pointers; async on `stream`. */
moe_status moe_pack_router(const moe_shape* shape, const void* w, const uint16_t* s,
                           const uint16_t* b, void* packed, size_t packed_bytes, void* stream);

/* ---------------------------------------------------------------- a1 + a2: routing
 * [P3-build] routing contract; parallel top-k router as in [P1-phase].
 * Inputs: router_packed (moe_pack_router layout); logit_bias [E] float or NULL,
 * added to the routed logits only; x [T][H] bf16.
 * Outputs: logits [T][R] float (fp32 logits; row-major; written first and then
 * read by the selection step), ids [T][k] int32 (descending logit, ties to the
 * lower id), w [T][k] bf16 (exp(l_i - l_0) / sum_j exp(l_j - l_0) over the picks,
 * evaluated in fp64 and rounded once), w_shared [T] bf16 (bf16(sigmoid(bf16(gate)))
 * in fp64; NULL when has_shared == 0). NaN logits rank below -inf; -0 ties +0.
 * Logits: for T <= 16 (and for the fp32 router) exact products accumulated in
 * fp64 in a fixed order and rounded once to fp32; for T > 16 with the 8-bit
 * router a matrix-core GEMM accumulating in fp32 (the 1e-5 near-tie allowance of
 * the pick check covers the difference). A token's logits do not depend on the
 * other tokens of the call. T >= 1. */
moe_status moe_route(const moe_shape* shape, const void* router_packed, const float* logit_bias,
                     const uint16_t* x, int32_t T, float* logits, int32_t* ids, uint16_t* w,
                     uint16_t* w_shared, void* stream);

/* The selection step alone, from caller-given fp32 logits [T][R] (same outputs). */
moe_status moe_route_from_logits(const moe_shape* shape, const float* logits, int32_t T,
                                 int32_t* ids, uint16_t* w, uint16_t* w_shared, void* stream);

/* ---------------------------------------------------------------- a4 + a5: experts, decode
 * GEMV path for 1 <= T <= 16 rows ([P1-phase]: the GEMV MoE path at batch 1;
 * [P3-build]: windows of 1 to 16 rows). For every token t and slot s with expert
 * e (ids[t,s], or the shared expert for s == k):
 *   h = bf16(silu(x Wg_e^T) * (x Wu_e^T))   (SwiGLU; the bf16 rounding is a reading)
 *   y[t][s][:] = h Wd_e^T                   (fp32, not rounded to bf16: [P3-build])
 * ws: device scratch of moe_decode_workspace_bytes(shape, T) bytes (holds h and,
 * for moe_decode_layer, its control words and the tagged logit and h words it
 * hands between workgroups). Each row's result does not depend on T
 * or on the other rows. Expert ids outside [0, E) give zero y rows. */
size_t moe_decode_workspace_bytes(const moe_shape* shape, int32_t T);
moe_status moe_experts_decode(const moe_shape* shape, const void* experts_packed,
                              const uint16_t* x, int32_t T, const int32_t* ids, void* ws,
                              size_t ws_bytes, float* y, void* stream);

/* moe_experts_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. The h rows go to a device array inside the
 * library (1,114,112 bytes: 16 tokens x 17 slots x 2048 intermediate values;
 * larger T * S * inter is refused with MOE_ERR_UNSUPPORTED), one per GPU, held
 * until the process ends. The call allocates nothing and gives the same y as
 * moe_experts_decode bit for bit. Every call on a GPU shares that GPU's array:
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race and must be ordered by the caller. Errors as moe_experts_decode. */
moe_status moe_experts_decode_noalloc(const moe_shape* shape, const void* experts_packed,
                                      const uint16_t* x, int32_t T, const int32_t* ids, float* y,
                                      void* stream);

/* The whole decode layer (1 <= T <= 16) in one launch: router logits, selection,
 * the gate/up GEMV with SwiGLU, and the down GEMV with the combine (same
 * arithmetic as moe_route, moe_experts_decode and moe_combine, so the outputs are
 * bit-identical to those three calls). Outputs: logits, ids, w, w_shared as moe_route; y [T][S][H] fp32
 * or NULL; out [T][H] bf16 (bf16(residual + out) if residual != NULL; residual
 * may alias out). One persistent launch (at most one workgroup per compute unit,
 * all resident): workgroups hand data to each other through words of ws tagged
 * with a per-launch epoch. ws belongs to one (shape, T): it must be zero-filled
 * before its first use with this call (and again before it is used with another
 * T) and is then ready for every later call without clearing; calls that share a
 * ws must not overlap in time, and the launch must not share the GPU with work
 * that keeps its workgroups from being resident (its waits are bounded: on a
 * timeout it sets an error word in ws and its outputs are undefined; see
 * moe_decode_layer_check). [P3-build], [P1-phase]. */
moe_status moe_decode_layer(const moe_shape* shape, const void* router_packed,
                            const float* logit_bias, const void* experts_packed,
                            const uint16_t* x, int32_t T, void* ws, size_t ws_bytes,
                            float* logits, int32_t* ids, uint16_t* w, uint16_t* w_shared,
                            float* y, const uint16_t* residual, uint16_t* out, void* stream);

/* One block of a layer stack in one launch: x_out = bf16(x + MoE(bf16(RMSNorm(x)))),
 * RMSNorm with unit weight and epsilon eps (>= 0): the layer runs on the
 * normalised tokens, and the residual add uses x as given (reading of the stack:
 * a pre-norm residual block, as moe_rmsnorm followed by moe_decode_layer with
 * residual = x; the outputs are bit-identical to those two calls). Arguments,
 * workspace, waits and errors as moe_decode_layer; logits, ids, w, w_shared and y
 * are the layer's; x_out [T][H] bf16 must not overlap x. [P3-build], [P1-phase]. */
moe_status moe_decode_block(const moe_shape* shape, const void* router_packed, const float* logit_bias,
                            const void* experts_packed, const uint16_t* x, int32_t T, float eps, void* ws,
                            size_t ws_bytes, float* logits, int32_t* ids, uint16_t* w, uint16_t* w_shared,
                            float* y, uint16_t* x_out, void* stream);

/* Waits for `stream`, then reads and clears the error word that moe_decode_layer
 * sets in ws (same shape and T) when one of its bounded waits times out. Returns
 * MOE_OK if no call since the last check timed out, MOE_ERR_TIMEOUT if one did
 * (the outputs of the calls since then are undefined), MOE_ERR_INVALID_ARG /
 * MOE_ERR_WORKSPACE for bad arguments, MOE_ERR_HIP if a runtime call fails. */
moe_status moe_decode_layer_check(const moe_shape* shape, int32_t T, void* ws, size_t ws_bytes,
                                  void* stream);

/* ---------------------------------------------------------------- a3: dispatch
 * Histogram and expert-sorted order of the T*S picks ([P1-phase] Phase 9b:
 * lookup-table dispatch). counts [M] int32 (counts[E] = T for the shared expert),
 * offsets [M+1] int32 exclusive prefix sums, order [T*S] int32: pick indices
 * p = t*S + s grouped by ascending expert; the order of picks inside one expert's
 * segment is unspecified (every valid order gives the same layer output). */
moe_status moe_dispatch(const moe_shape* shape, const int32_t* ids, int32_t T, int32_t* counts,
                        int32_t* offsets, int32_t* order, void* stream);

/* ---------------------------------------------------------------- a3..a5: experts, prefill
 * Grouped-GEMM path for any T >= 1 ([P1-phase] Phase 9b: MoE GEMM with int4
 * dequant and dispatch table). Same y as moe_experts_decode up to fp32
 * summation order. Runs moe_dispatch internally into `ws`, then the gate/up GEMM
 * with the SwiGLU epilogue, then the down GEMM scattering rows back to y[t][s].
 * experts_prefill: the prefill layout that moe_pack_experts_prefill wrote (not the
 * packed buffer itself). ws: device scratch of moe_prefill_workspace_bytes(shape, T)
 * bytes. */
size_t moe_prefill_workspace_bytes(const moe_shape* shape, int32_t T);

/* The prefill layout of packed experts: the same bytes as moe_pack_experts' buffer
 * (moe_experts_packed_bytes), permuted within each set of 64 consecutive four-row
 * blocks of a matrix (the last set of a matrix may hold fewer, n): the 128-byte
 * line of block j and group g of a set moves from set + 128 (j G + g) to
 * set + 128 (g n + j), G groups per row, and its 16-byte (scale, bias) unit from
 * sb set + 16 (j G + g) to sb set + 16 (g n + j). One grouped-GEMM workgroup reads
 * one set, one group at a time, so each chunk is one contiguous run of memory.
 * Reads experts_packed (device, moe_pack_experts' layout) and writes
 * experts_prefill (device, bytes >= moe_experts_packed_bytes; the two must not
 * overlap). Async on `stream`. MOE_ERR_WORKSPACE if bytes is too small. */
moe_status moe_pack_experts_prefill(const moe_shape* shape, const void* experts_packed, void* experts_prefill,
                                    size_t bytes, void* stream);

/* Where moe_experts_prefill leaves its dispatch inside ws for a call with this
 * shape and T (byte offsets from ws; written to *view_host, host memory):
 *   counts [M] int32 (counts[E] = T for the shared expert), offsets [M+1] int32
 *   (exclusive prefix sums), ntiles one int32, tiles [max_tiles] of four int32
 *   {expert, row0, nrows, 0} (the first ntiles are the work list: a tile covers
 *   rows row0 .. row0+nrows-1 of the expert-sorted order, at most tile_rows, all of
 *   one expert), order [T*S] int32 (pick indices t*S + s grouped by ascending expert,
 *   and within an expert by ascending pick index).
 * For checks of the dispatch and for callers that reuse the expert-sorted order
 * ([P1-phase] Phase 9b: lookup-table dispatch). MOE_ERR_INVALID_ARG for a bad
 * shape, T < 1 or NULL view_host. */
typedef struct moe_prefill_dispatch_view {
    size_t counts, offsets, ntiles, tiles, order;
    int32_t max_tiles;
    int32_t tile_rows;  /* the tiles' height: 64 for T <= 1024, else 128 */
} moe_prefill_dispatch_view;
moe_status moe_prefill_dispatch_layout(const moe_shape* shape, int32_t T, moe_prefill_dispatch_view* view_host);

moe_status moe_experts_prefill(const moe_shape* shape, const void* experts_prefill,
                               const uint16_t* x, int32_t T, const int32_t* ids, void* ws,
                               size_t ws_bytes, float* y, void* stream);

/* ---------------------------------------------------------------- FP8 route (prefill)
 * [P2-next]: the experts upcast once to FP8 so the prompt GEMMs run on the FP8
 * matrix cores. Not exact: every operand carries one FP8 rounding (about 6 % rms
 * relative error on the layer output); the routing, dispatch and combine are the
 * exact path's. Format (OCP FP8 E4M3, round to nearest even, no saturation):
 *   - weight row (gate, up or down, of the canonical 4- or 8-bit expert): w =
 *     fp32(scale * q + bias) (one rounding: a fused multiply-add), e = floor(log2
 *     max|w|) - 7 (0 for an all-zero row), codes = E4M3(w * 2^-e), so the row's
 *     largest magnitude maps into [128, 256); the row scale 2^e is kept as a float;
 *   - activation rows entering a projection (x for gate/up, the bf16 SwiGLU
 *     intermediate h for down) are quantised the same way, one 2^e per row;
 *   - a projection output is the fp32 sum of code products times both rows' 2^e;
 *     h = bf16(silu(gate) * up) as in the exact path.
 * FP8 buffer, per expert m (stride = moe_experts_fp8_bytes / M, 256-byte aligned):
 *   gate codes [I][Hp] | up codes [I][Hp] | down codes [H][Ip] |
 *   row scales float [2I + H] (gate rows, up rows, down rows),
 * Hp = H and Ip = I rounded up to multiples of 128, padding codes 0. */
size_t moe_experts_fp8_bytes(const moe_shape* shape);

/* Upcasts canonical experts (device arrays, 4- or 8-bit as shape->bits says, codes
 * 8-byte aligned) into `fp8` (device, 256-byte aligned, fp8_bytes >=
 * moe_experts_fp8_bytes). Async on `stream`. */
moe_status moe_pack_experts_fp8(const moe_shape* shape, const moe_expert_canon* src_host,
                                void* fp8, size_t fp8_bytes, void* stream);

/* moe_experts_prefill's contract (y [T][S][H] fp32, per-slot expert outputs; rows
 * of picks with an id outside [0, E) zeroed) through the FP8 route: dispatch with
 * tiles of up to 128 rows, x quantised per row, the FP8 gate/up GEMM writing h, h
 * quantised per row, the FP8 down GEMM. Each output depends on its own token's row
 * only, in a fixed order (any T, any call). ws: device scratch of
 * moe_prefill_fp8_workspace_bytes(shape, T) bytes (its layout is internal).
 * MOE_ERR_UNSUPPORTED when
 * T * Hp or T * S * Ip reaches 2^32 or the device has under 76 KiB of LDS per
 * workgroup. */
size_t moe_prefill_fp8_workspace_bytes(const moe_shape* shape, int32_t T);
moe_status moe_experts_prefill_fp8(const moe_shape* shape, const void* experts_fp8,
                                   const uint16_t* x, int32_t T, const int32_t* ids, void* ws,
                                   size_t ws_bytes, float* y, void* stream);

/* ---------------------------------------------------------------- a6: combine
 * out[t][n] = bf16( sum_{s<k} w[t][s] * y[t][s][n] + w_shared[t] * y[t][k][n] )
 * with one rounding ([P3-build]); fp32 sum in slot order. If residual != NULL
 * (a [T][H] bf16 array, may alias out) the result is bf16(residual + that value):
 * the residual add of a stacked block. w_shared must be NULL iff has_shared == 0. */
moe_status moe_combine(const moe_shape* shape, const float* y, const uint16_t* w,
                       const uint16_t* w_shared, int32_t T, const uint16_t* residual,
                       uint16_t* out, void* stream);

/* ---------------------------------------------------------------- a7: stack glue
 * Unit-weight RMSNorm per row: out = bf16(x * r), r = 1 / sqrt(mean(x^2) + eps) in
 * fp32; the sum of squares runs in one fixed order (the one moe_decode_block uses).
 * (Reading: the pages give no norm for an MoE-only stack; a pre-norm residual block
 * x <- x + MoE(RMSNorm(x)) keeps stacked activations in range.) out may not alias x. */
moe_status moe_rmsnorm(int32_t hidden, const uint16_t* x, int32_t T, float eps, uint16_t* out,
                       void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
