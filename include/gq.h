/*
 * gq.h -- C ABI of libgq: grouped mixture-of-experts matmul on 4-bit packed
 * expert weights (NF4 and MXFP4) for AMD MI355X (gfx950).
 *
 * What the library computes follows these web pages:
 *   [P1] "grouped-nf4-gemm 0.43.0" (PyPI project page): section "Which
 *        entry point?" (grouped NF4 forward and backward, the single-row
 *        decode bandwidth route, native MXFP4 expert math) and the page
 *        header (one GPU launch for the active experts, no full-size bf16
 *        weight copies); section "Try the packers and byte checks on CPU"
 *        (packed shapes).
 *   [P2] "Receipts-driven engineering": opening summary (codebook decoded
 *        in registers inside the GEMM mainloop; NF4 in the bitsandbytes
 *        packed layout; MXFP4 as OCP e2m1 on released bytes; the NF4 path
 *        is differentiable).
 *   [P4] "flashrt/grouped-moe-gemv": section "Functions" (routing tensor
 *        [M, top_k] of expert ids, output [M, top_k, N], flatten to
 *        M = routed pairs and top_k = 1 when each pair has its own input;
 *        no atomics, no host synchronisation, caller-owned buffers).
 *   [P5] GPTQModel wiki "NF12": malformed arguments to native C-ABI calls
 *        return hipErrorInvalidValue; launches beyond supported limits
 *        return hipErrorNotSupported before launch.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every buffer pointer is DEVICE memory on the current HIP device and is
 *   owned by the caller; the library never allocates, frees or keeps a
 *   pointer after the call returns.
 * - Work is enqueued asynchronously on `stream` (NULL = default stream);
 *   nothing synchronises the host.  Results are ready when the stream is.
 * - bf16 values travel as raw uint16_t bit patterns.
 * - Packed weights (all experts stacked, contiguous):
 *     NF4   codes  uint8 [E, N, K/2]  element 2j of a row in the HIGH nibble
 *                                     of byte j (bitsandbytes layout)
 *           absmax float [E, N, K/64] one scale per 64 consecutive k
 *           weight = float32(nf4_codebook[code] * absmax)
 *     MXFP4 blocks uint8 [E, N, K/32, 16] element 2j of a 32-block in the LOW
 *                                     nibble of byte j (released gpt-oss layout)
 *           scales uint8 [E, N, K/32] e8m0: factor 2^(s-127); 255 = NaN
 *           weight = e2m1(code) * 2^(s-127)
 * - Routing: topk_ids int32 [rows, topk], pair index p = t*topk + s.  A pair
 *   routed to an id outside [0, E) is dropped and its output row is zeros.
 *   Gather mode (topk > 1): pair p reads activation row p / topk.  Flatten
 *   mode (per-pair inputs, e.g. a down projection): pass rows = pairs and
 *   topk = 1.
 * - Outputs are bf16, rounded to nearest even from an fp32 accumulator,
 *   optionally multiplied by pair_scale[p] (fp32, one per pair; NULL = 1).
 *   No atomics: each output element is written by exactly one thread, so
 *   results are bitwise reproducible run to run.
 * - Return value: 0 on success; hipErrorInvalidValue (1) for a malformed
 *   argument (checked on the host before anything is enqueued; nothing is
 *   truncated or clamped); hipErrorNotSupported (801) for a well-formed
 *   request outside what the kernels support (stated per function);
 *   otherwise the HIP error reported by the launch.
 * - Expert ids are data on the device; the kernels treat any id outside
 *   [0, E) as dropped, so no id can make a kernel read outside the banks.
 */
#ifndef GQ_H
#define GQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Name of a status code returned by this library (static string). */
const char* gq_status_string(int status);

/* ------------------------------------------------------------------------
 * Token-to-expert grouping.  [P1] header and [P2] summary: all active
 * experts run in one launch, which needs the pairs grouped by expert on the
 * device without a host round trip ([P4] "Functions": no host sync).
 *
 * Upper bound on the number of tiles gq_route_sort can emit, including the
 * tiles the grouped GEMM uses to clear dropped rows:
 *     ceil(rows*topk / tile_m) + E + 1.
 * Returns -1 if an argument is negative, tile_m < 1 or E < 1.
 */
int32_t gq_route_max_tiles(int32_t rows, int32_t topk, int32_t num_experts, int32_t tile_m);

/*
 * Stable counting sort of the rows*topk (token, slot) pairs by expert.
 *   topk_ids       int32 [rows, topk]       in
 *   expert_offsets int32 [E + 1]            out: offsets[e] = #valid pairs with
 *                                                expert < e; offsets[E] = #valid pairs
 *   sorted_pairs   int32 [rows*topk]        out: expert by expert, ascending pair
 *                                                index within an expert; dropped
 *                                                pairs last, ascending
 *   tiles          int32 [max_tiles, 2]     out: (expert, start in sorted_pairs) of
 *                                                every tile_m-row slice of each
 *                                                expert's segment, experts
 *                                                ascending; unused entries = -1
 *   num_tiles      int32 [1]                out: number of valid tiles
 * Deterministic: the output is the unique answer to the definition above.
 * InvalidValue: null pointer, rows/topk < 0, E < 1, tile_m < 1,
 *               max_tiles < gq_route_max_tiles(...).
 * NotSupported: E > 1024, rows*topk >= 2^31.
 * rows*topk == 0 is valid (offsets all 0, num_tiles 0, tiles all -1).
 */
int gq_route_sort(const int32_t* topk_ids, int32_t rows, int32_t topk, int32_t num_experts,
                  int32_t tile_m, int32_t* expert_offsets, int32_t* sorted_pairs,
                  int32_t* tiles, int32_t max_tiles, int32_t* num_tiles, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode probes.  [P1] "Try the packers and byte checks on CPU" (packed
 * shapes) and [P2] summary (codes decoded in registers).  They write the
 * decoded weights with the same device decode routines the matmul kernels
 * use, so decoding can be compared bit for bit.  Not on the hot path.
 *   NF4:   codes [n_rows, K/2], absmax [n_rows, K/64]; K % 64 == 0
 *   MXFP4: blocks [n_rows, K/32, 16], scales [n_rows, K/32]; K % 32 == 0
 *   out_f32 float [n_rows, K] (may be NULL), out_bf16 uint16 [n_rows, K]
 *   (may be NULL; bf16 = RNE of the float32 weight).  At least one output.
 * InvalidValue: null inputs, both outputs NULL, n_rows < 0, K <= 0 or not a
 * multiple of the block.
 */
int gq_nf4_decode(const uint8_t* codes, const float* absmax, int64_t n_rows, int32_t K,
                  float* out_f32, uint16_t* out_bf16, hipStream_t stream);
int gq_mxfp4_decode(const uint8_t* blocks, const uint8_t* scales, int64_t n_rows, int32_t K,
                    float* out_f32, uint16_t* out_bf16, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Decode-time GEMV: 1..8 tokens in gather mode, or their routed pairs in
 * flatten mode (at most 256 pairs).  [P1] header, "Which entry point?"
 * (single-row decode bandwidth route), [P4] "Functions" (one product per
 * routed slot, [M, top_k] -> [M, top_k, N]).
 *
 *   out[p, n] = bf16( pair_scale[p] * sum_k x[p/topk, k] * W_{ids[p]}[n, k] )
 *
 *   x          uint16 bf16 [rows, K] with row stride x_stride elements
 *              (x_stride >= K, x_stride % 8 == 0, x 16-byte aligned)
 *   codes/absmax (NF4) or blocks/scales (MXFP4) for E experts of shape [N, K]
 *   topk_ids   int32 [rows, topk]; pair_scale float [rows*topk] or NULL
 *   out        uint16 bf16 [rows*topk, N]
 * Each distinct active expert's bytes are read once, whichever tokens use
 * it; no sort is needed (the kernel reads topk_ids directly).  Arithmetic,
 * float32 throughout with no bf16 rounding of the weights: each group of 32
 * consecutive k is summed as sum(codebook_value * x) (NF4) or
 * sum(e2m1_value * x) (MXFP4; exact products, two per bf16-pair dot
 * instruction, float32 sums), then multiplied once by the group's factor
 * (the NF4 absmax of its 64-block; the MXFP4 2^(s-127), exact); the group
 * partials are added in a fixed order.  A one-hot x therefore returns
 * bf16(float32(value * factor)), the decoded weight, bit for bit.
 * InvalidValue: null pointer (pair_scale may be NULL), rows < 1,
 *   topk < 1, E < 1, N < 1, K not a positive multiple of 64 (NF4) / 32
 *   (MXFP4), bad stride or alignment.
 * A pair whose id lies outside [0, E) is dropped: its output row is zero.
 * NotSupported: rows*topk > 256, K > 8192, N >= 2^24, N*K/2 >= 2^31 (one
 *   expert's codes), x_stride > 2^31 - 1.
 */
int gq_nf4_grouped_gemv(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                        const uint8_t* codes, const float* absmax, int32_t num_experts,
                        int32_t N, const int32_t* topk_ids, int32_t topk,
                        const float* pair_scale, uint16_t* out, hipStream_t stream);
int gq_mxfp4_grouped_gemv(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                          const uint8_t* blocks, const uint8_t* scales, int32_t num_experts,
                          int32_t N, const int32_t* topk_ids, int32_t topk,
                          const float* pair_scale, uint16_t* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Experts streamed from host memory.  [P1] page header (streaming expert
 * weights from RAM or SSD) and section "Which entry point?" (the row for
 * streaming experts from RAM or NVMe); [P2] "What the discipline caught" (the fused
 * kernel as the only expert compute while experts stream over the host
 * link, against the link's ceiling) and "The numbers" (t ~ c + bytes/link).
 *
 * gq_nf4_grouped_gemv_host / gq_mxfp4_grouped_gemv_host: gq_nf4_grouped_gemv
 * / gq_mxfp4_grouped_gemv with the expert bank (codes and absmax, or blocks
 * and scales) in pinned, device-mapped host memory (hipHostMalloc, or a
 * pinned torch tensor), passed as HOST pointers.  The kernel reads the
 * routed experts' bytes straight over the host link as it decodes them: no
 * staging copy, each active expert's bytes cross the link once per launch.
 * x, topk_ids, pair_scale and out are device pointers as before; same
 * arithmetic, results bit-identical to the device-resident call.
 * InvalidValue also when a bank pointer is not pinned, mapped host memory
 * (checked before anything is enqueued).
 */
int gq_nf4_grouped_gemv_host(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                             const uint8_t* codes, const float* absmax, int32_t num_experts,
                             int32_t N, const int32_t* topk_ids, int32_t topk,
                             const float* pair_scale, uint16_t* out, hipStream_t stream);
int gq_mxfp4_grouped_gemv_host(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                               const uint8_t* blocks, const uint8_t* scales, int32_t num_experts,
                               int32_t N, const int32_t* topk_ids, int32_t topk,
                               const float* pair_scale, uint16_t* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Prefill grouped GEMM.  [P1] "Which entry point?" (grouped NF4 forward,
 * native MXFP4 expert math) and header (one launch for the active experts,
 * no full-size bf16 weight copies); [P2] summary (codebook decoded in
 * registers inside the mainloop).
 *
 *   out[p, n] = bf16( pair_scale[p] * sum_k x[p/topk, k] * W_{ids[p]}[n, k] )
 *
 * Same x / weights / pair_scale / out conventions as the GEMV.  The
 * grouping comes from gq_route_sort(topk_ids, rows, topk, E, tile_m, ...)
 * called with the same tile_m: expert_offsets, sorted_pairs, tiles,
 * num_tiles and max_tiles are passed through unchanged.  Dropped pairs'
 * rows are written as zeros by the same launch.  Arithmetic: decoded weight
 * rounded to bf16 (NF4: RNE of the float32 weight; MXFP4: exact), bf16
 * matrix-core products, float32 accumulation.
 * InvalidValue: null pointer (pair_scale may be NULL), rows < 0, topk < 1,
 *   E < 1, N < 1 or N % 32, K not a positive multiple of 64 (NF4) / 32
 *   (MXFP4), bad stride or alignment, max_tiles below the bound.
 * NotSupported: tile_m != 256, rows*topk >= 2^31, grid beyond 2^31 blocks.
 * rows == 0 enqueues nothing.
 */
int gq_nf4_grouped_gemm(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                        const uint8_t* codes, const float* absmax, int32_t num_experts,
                        int32_t N, int32_t topk, const float* pair_scale,
                        const int32_t* expert_offsets, const int32_t* sorted_pairs,
                        const int32_t* tiles, const int32_t* num_tiles, int32_t max_tiles,
                        int32_t tile_m, uint16_t* out, hipStream_t stream);
int gq_mxfp4_grouped_gemm(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                          const uint8_t* blocks, const uint8_t* scales, int32_t num_experts,
                          int32_t N, int32_t topk, const float* pair_scale,
                          const int32_t* expert_offsets, const int32_t* sorted_pairs,
                          const int32_t* tiles, const int32_t* num_tiles, int32_t max_tiles,
                          int32_t tile_m, uint16_t* out, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MXFP4 prefill on the block-scaled fp4 matrix instruction.  [P2] summary
 * (MXFP4 as OCP e2m1 on the checkpoint's released bytes, decoded inside the
 * mainloop); [P3] summary (native MXFP4 expert inference); [P1] "Which
 * entry point?" (native MXFP4 expert math).  The weights' e2m1 codes and
 * e8m0 scales are fed to the gfx950 instruction as stored, with no decode.
 * The pages keep activations in bf16; the instruction's other operand must
 * be an MX format too, so the activations are first written as two e4m3
 * terms (the reading of this library):
 *
 *   x[t, k] ~= hi[t, k] * 2^(s_hi[t, k/32] - 127) + lo[t, k] * 2^(s_lo[t, k/32] - 127)
 *
 * per 32 consecutive k: X = the smallest integer with amax * 2^-X <= 448
 * (the largest e4m3 magnitude; -127 for an all-zero block), hi = e4m3 of
 * x * 2^-Xh rounded to nearest even, lo the same for the exact residual
 * x - hi * 2^Xh with its own exponent.  The two terms hold every bf16 value
 * of a block exactly unless its magnitudes span 2^12 or more; in any case
 * |x - split| <= 2^-8 |x| + 2^-16 amax.  Results are then within the same
 * tolerance of the float64 W4A16 product as the bf16 path.
 *
 * gq_act_split_e4m3: x uint16 bf16 [rows, K] (row stride x_stride elements,
 * a multiple of 8; K a multiple of 32) -> with Kp = K rounded up to 64:
 *   codes  uint8 [rows, 2*Kp]: per row and 64-k step s, 128 bytes: hi codes
 *          then lo codes, 64 bytes each; in each, bytes [32h, 32h+32) hold
 *          elements 16h + [0, 16) of k block 2s, then of block 2s+1 (the
 *          order the instruction's e4m3 operand takes them in)
 *   scales uint8 [rows, Kp/16]: per step s_hi(2s), s_lo(2s), s_hi(2s+1),
 *          s_lo(2s+1)
 * A block past K (K % 64 == 32) is written as zeros with scale byte 0.
 * codes 16-byte aligned, scales 4-byte aligned.
 * InvalidValue: null pointer, rows < 0, K not a positive multiple of 32,
 *   bad stride or alignment.  NotSupported: grid beyond 2^31 blocks.
 *
 * gq_mxfp4_grouped_gemm_scaled: as gq_mxfp4_grouped_gemm with the
 * activations given as gq_act_split_e4m3's output for x [rows, K]:
 *
 *   out[p, n] = bf16( pair_scale[p] * sum_k split(x)[p/topk, k] * W_{ids[p]}[n, k] )
 *
 * float32 accumulation.  Same grouping, pair_scale and out conventions.
 * InvalidValue: null pointer (pair_scale may be NULL), rows < 0, topk < 1,
 *   E < 1, N < 1 or N % 32, K not a positive multiple of 32, bad alignment,
 *   max_tiles below the bound.
 * NotSupported: tile_m != 256, rows*topk >= 2^31, rows*2*Kp >= 2^31, grid
 *   beyond 2^31 blocks.  rows == 0 enqueues nothing.
 *
 * gq_mxfp4_grouped_gemm_scaled_swiglu: the gate_up product of gpt-oss's
 * experts with their gated unit applied in the epilogue.  The pages run
 * gpt-oss MXFP4 experts ("Receipts-driven engineering", "The numbers") but
 * do not define the activation; the reading of this library is gpt-oss's
 * published expert MLP, whose fused gate_up weight interleaves gate row j
 * (row 2j) and up row j (row 2j + 1):
 *
 *   g = sum_k split(x)[p/topk, k] * W[2j, k],  u = ... W[2j + 1, k]
 *   act[p, j] = bf16( gc * sigmoid(alpha * gc) * (uc + 1) ),
 *   gc = min(g, limit),  uc = min(max(u, -limit), limit)
 *
 * in float32, sigmoid(z) = 1 / (1 + 2^(-z log2 e)) from the hardware
 * exponential and reciprocal (a few float32 ulp; gpt-oss: alpha = 1.702,
 * limit = 7).  blocks/scales [E, N, K]
 * with N = 2I; act uint16 bf16 [rows*topk, I], rows of dropped pairs zero.
 * No pair_scale.  Errors as gq_mxfp4_grouped_gemm_scaled, plus
 * InvalidValue for a non-finite alpha or limit, or limit < 0.
 *
 * gq_mxfp4_grouped_gemm_scaled_swiglu_split: the same product and gated
 * unit, the bf16 result written as its two-term e4m3 split (the layout of
 * gq_act_split_e4m3 for [rows*topk, I]) instead of as bf16, so that it
 * feeds the down product directly:
 *
 *   act_codes, act_scales = gq_act_split_e4m3(act)   (bytes identical)
 *
 * act_codes uint8 [rows*topk, 2I] (16-byte aligned), act_scales uint8
 * [rows*topk, I/16] (4-byte aligned); rows of dropped pairs get zero codes
 * and zero scale bytes (the split of a zero row).  Errors as
 * gq_mxfp4_grouped_gemm_scaled_swiglu; NotSupported also when N % 128 != 0
 * (I a multiple of 64: whole 64-column split steps).
 */
int gq_act_split_e4m3(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                      uint8_t* codes, uint8_t* scales, hipStream_t stream);
int gq_mxfp4_grouped_gemm_scaled(const uint8_t* x_codes, const uint8_t* x_scales, int32_t rows,
                                 int32_t K, const uint8_t* blocks, const uint8_t* scales,
                                 int32_t num_experts, int32_t N, int32_t topk,
                                 const float* pair_scale, const int32_t* expert_offsets,
                                 const int32_t* sorted_pairs, const int32_t* tiles,
                                 const int32_t* num_tiles, int32_t max_tiles, int32_t tile_m,
                                 uint16_t* out, hipStream_t stream);
int gq_mxfp4_grouped_gemm_scaled_swiglu(const uint8_t* x_codes, const uint8_t* x_scales,
                                        int32_t rows, int32_t K, const uint8_t* blocks,
                                        const uint8_t* scales, int32_t num_experts, int32_t N,
                                        int32_t topk, float alpha, float limit,
                                        const int32_t* expert_offsets,
                                        const int32_t* sorted_pairs, const int32_t* tiles,
                                        const int32_t* num_tiles, int32_t max_tiles,
                                        int32_t tile_m, uint16_t* act, hipStream_t stream);
int gq_mxfp4_grouped_gemm_scaled_swiglu_split(
    const uint8_t* x_codes, const uint8_t* x_scales, int32_t rows, int32_t K,
    const uint8_t* blocks, const uint8_t* scales, int32_t num_experts, int32_t N, int32_t topk,
    float alpha, float limit, const int32_t* expert_offsets, const int32_t* sorted_pairs,
    const int32_t* tiles, const int32_t* num_tiles, int32_t max_tiles, int32_t tile_m,
    uint8_t* act_codes, uint8_t* act_scales, hipStream_t stream);

/* ------------------------------------------------------------------------
 * NF4 input gradient.  [P1] "Which entry point?" (grouped NF4 backward);
 * [P2] summary (the NF4 path is differentiable, fine-tuning stays packed).
 *
 *   dx[p, k] = bf16( sum_n dy[p, n] * W_{e(p)}[n, k] )
 *
 *   dy   uint16 bf16 [P, N] with row stride dy_stride elements (per pair)
 *   dx   uint16 bf16 [P, K]
 * The grouping comes from gq_route_sort(pair_expert, P, 1, E, tile_m, ...);
 * pairs with an expert outside [0, E) get dx rows of zeros.  Same decode
 * and arithmetic as the NF4 GEMM, contraction over N.
 * InvalidValue: null pointer, P < 0, E < 1, N < 1 or N % 64, K not a
 *   positive multiple of 64, bad stride or alignment, max_tiles too small.
 * NotSupported: tile_m != 256, grid beyond 2^31 blocks.
 */
int gq_nf4_grouped_dgrad(const uint16_t* dy, int32_t P, int32_t N, int64_t dy_stride,
                         const uint8_t* codes, const float* absmax, int32_t num_experts,
                         int32_t K, const int32_t* expert_offsets, const int32_t* sorted_pairs,
                         const int32_t* tiles, const int32_t* num_tiles, int32_t max_tiles,
                         int32_t tile_m, uint16_t* dx, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MXFP4 input gradient.  [P1] "Which entry point?" (native MXFP4 expert
 * math next to the grouped NF4 backward).  The pages name no MXFP4
 * backward entry point; this is the NF4 one with the MXFP4 decode:
 *
 *   dx[p, k] = bf16( sum_n dy[p, n] * W_{e(p)}[n, k] )
 *
 *   blocks  uint8 [E, N, K/32, 16] e2m1 codes (element 2j: low nibble)
 *   scales  uint8 [E, N, K/32] e8m0 (255 = NaN)
 * Decoded weights are exact in bf16; bf16 matrix-core products, float32
 * accumulation.  dy, dx and the grouping as for gq_nf4_grouped_dgrad.
 * InvalidValue: null pointer, P < 0, E < 1, N < 1 or N % 64, K not a
 *   positive multiple of 32, bad stride or alignment, max_tiles too small.
 * NotSupported: tile_m != 256, grid beyond 2^31 blocks.
 */
int gq_mxfp4_grouped_dgrad(const uint16_t* dy, int32_t P, int32_t N, int64_t dy_stride,
                           const uint8_t* blocks, const uint8_t* scales, int32_t num_experts,
                           int32_t K, const int32_t* expert_offsets, const int32_t* sorted_pairs,
                           const int32_t* tiles, const int32_t* num_tiles, int32_t max_tiles,
                           int32_t tile_m, uint16_t* dx, hipStream_t stream);

/* ------------------------------------------------------------------------
 * MoE-layer epilogues.  The pages benchmark the grouped products on the
 * Qwen3-30B-A3B expert shapes, whose experts are SwiGLU MLPs; [P1] header
 * (one launch for the active experts) and [P4] "Functions" ([M, top_k]
 * routing, per-slot [M, top_k, N] outputs that the caller reduces over
 * top_k).  The pages leave the activation and the reduction to the caller;
 * these entry points fuse them (readings: gate rows [0, I) then up rows
 * [I, 2I) in a fused gate_up weight; SwiGLU act = silu(gate) * up with
 * silu(z) = z / (1 + exp(-z)); combine = router-weighted sum over a
 * token's slots, in slot order).  All arithmetic float32, one bf16
 * rounding per output; sigmoid (in silu and in gpt-oss's gated unit) is
 * 1 / (1 + 2^(-z log2 e)) from the hardware exponential and reciprocal, a
 * few float32 ulp from the correctly rounded value.
 *
 * gq_nf4_grouped_gemv_swiglu / gq_nf4_grouped_gemm_swiglu:
 *   act[p, j] = bf16( silu(g) * u ),  g = sum_k x[p/topk, k] * W[j, k],
 *                                     u = sum_k x[p/topk, k] * W[I + j, k]
 *   codes/absmax [E, N, K] with N = 2I; act uint16 bf16 [rows*topk, I].
 *   Arguments, grouping and errors as gq_nf4_grouped_gemv / _gemm without
 *   pair_scale; InvalidValue also for N odd (GEMV) or N % 64 (GEMM).
 *
 * gq_mxfp4_grouped_gemv_swiglu: the decode gate_up GEMV of gpt-oss's
 * experts with their gated unit (the gq_mxfp4_grouped_gemm_scaled_swiglu
 * reading: gate row 2j, up row 2j + 1, act = gc * sigmoid(alpha * gc) *
 * (uc + 1), gc = min(g, limit), uc = min(max(u, -limit), limit)), on the
 * exact float32 products of gq_mxfp4_grouped_gemv.  blocks/scales
 * [E, N, K] with N = 2I; act uint16 bf16 [rows*topk, I].  Errors as
 * gq_mxfp4_grouped_gemv without pair_scale, plus InvalidValue for N odd, a
 * non-finite alpha or limit, or limit < 0.
 *
 * gq_nf4_grouped_gemv_down_combine (decode, rows*topk <= 64):
 *   y[t, n] = bf16( sum_s w[t, s] * sum_i act[t*topk + s, i] * W_{ids[t, s]}[n, i] )
 *   act   uint16 bf16 [rows*topk, I], row stride act_stride elements
 *   codes/absmax [E, H, I] NF4 (I % 64 == 0); topk_weights float [rows, topk]
 *   or NULL (weights 1); y uint16 bf16 [rows, H].  A slot whose expert is
 *   outside [0, E) contributes 0.
 *   InvalidValue: null pointer (topk_weights may be NULL), rows < 1,
 *     topk < 1, E < 1, H < 1, I not a positive multiple of 64, bad stride
 *     or alignment.  NotSupported: rows*topk > 64, I > 4096, I > 2048 with
 *     rows*topk > 32, H >= 2^24, act_stride > 2^31 - 1.
 *
 * gq_mxfp4_grouped_gemv_down_combine: the same on MXFP4 experts
 *   (blocks/scales [E, H, I], I a positive multiple of 32), float32 exact
 *   decode as gq_mxfp4_grouped_gemv; same errors with I % 32 for I % 64.
 *
 * gq_moe_combine (prefill):
 *   y[t, :] = bf16( sum_s w[t, s] * y_pairs[t*topk + s, :] )
 *   y_pairs uint16 bf16 [rows*topk, H] (row stride `stride` elements);
 *   topk_weights float [rows, topk] or NULL (plain sum, e.g. when the
 *   router weight was applied as pair_scale); y uint16 bf16 [rows, H].
 *   InvalidValue: rows < 0, topk < 1, H < 1 or H % 8, stride < H or
 *   stride % 8, null or misaligned pointers.  rows == 0 enqueues nothing.
 */
int gq_nf4_grouped_gemv_swiglu(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                               const uint8_t* codes, const float* absmax, int32_t num_experts,
                               int32_t N, const int32_t* topk_ids, int32_t topk, uint16_t* act,
                               hipStream_t stream);
int gq_nf4_grouped_gemm_swiglu(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                               const uint8_t* codes, const float* absmax, int32_t num_experts,
                               int32_t N, int32_t topk, const int32_t* expert_offsets,
                               const int32_t* sorted_pairs, const int32_t* tiles,
                               const int32_t* num_tiles, int32_t max_tiles, int32_t tile_m,
                               uint16_t* act, hipStream_t stream);
int gq_mxfp4_grouped_gemv_swiglu(const uint16_t* x, int32_t rows, int32_t K, int64_t x_stride,
                                 const uint8_t* blocks, const uint8_t* scales,
                                 int32_t num_experts, int32_t N, const int32_t* topk_ids,
                                 int32_t topk, float alpha, float limit, uint16_t* act,
                                 hipStream_t stream);
int gq_nf4_grouped_gemv_down_combine(const uint16_t* act, int32_t rows, int32_t I,
                                     int64_t act_stride, const uint8_t* codes,
                                     const float* absmax, int32_t num_experts, int32_t H,
                                     const int32_t* topk_ids, int32_t topk,
                                     const float* topk_weights, uint16_t* y,
                                     hipStream_t stream);
int gq_mxfp4_grouped_gemv_down_combine(const uint16_t* act, int32_t rows, int32_t I,
                                       int64_t act_stride, const uint8_t* blocks,
                                       const uint8_t* scales, int32_t num_experts, int32_t H,
                                       const int32_t* topk_ids, int32_t topk,
                                       const float* topk_weights, uint16_t* y,
                                       hipStream_t stream);
int gq_moe_combine(const uint16_t* y_pairs, int32_t rows, int32_t topk, int32_t H,
                   int64_t stride, const float* topk_weights, uint16_t* y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GQ_H */
