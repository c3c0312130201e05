/*
 * moe.h -- C ABI of the MoE expert layer for MI355X (gfx950).
 *
 * One MoE layer on one GPU: fp32 router logits -> top-k route -> align
 * (stable counting sort of token-expert pairs into per-expert segments padded
 * to the GEMM tile, with the expert -> slot indirection) -> per-expert SwiGLU
 * FFN reading FP8 or int4 expert weights from a per-layer VRAM slot pool ->
 * weighted combine.
 *
 * Sources (web pages, cited by title and section):
 *  [PW]  "PagedWeight: Efficient MoE LLM Serving with Dynamic Quality-Aware
 *        Weight Quantization", spectral-agent.com commentary.
 *  [MG]  MOE-GEN explainer, aibr.jp.
 *  [VEP] "vllm-expert-pager" article, rand.pepabo.com.
 *
 * Conventions for every call:
 *  - Pointers named d_* are device memory owned by the caller; the library
 *    borrows them for the call and keeps no reference afterwards.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *    is the default stream). They never synchronise and never allocate device
 *    memory; scratch memory is the caller's workspace argument.
 *  - Return MOE_OK (0) or a negative status. MOE_EINVAL: a host-side argument
 *    is invalid (null pointer, size out of range, workspace too small);
 *    nothing was launched. MOE_EHIP: a launch failed; moe_last_hip_error()
 *    gives the hipError_t value.
 *  - Problems only the device can see are added to the caller's int32 error
 *    word d_err (the caller zeroes it); the pairs concerned contribute zero
 *    to the output and the call still completes.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

enum { MOE_OK = 0, MOE_EINVAL = -1, MOE_EHIP = -2, MOE_ESCRATCH = -3 };

/* Slot storage formats ([PW] "technically interesting points": each expert is
 * held at its own bit width; [VEP] introduction: official FP8 weights). */
enum { MOE_FMT_FP8_E4M3_ROW = 0, /* OCP e4m3fn codes, one fp32 scale per row   */
       MOE_FMT_INT4_G128 = 1 };  /* uint4, fp16 (scale, zero) per 128 along K */

/* Activation precision of the expert FFN (the pages fix none):
 *  MOE_ACT_BF16: token rows enter the contraction exactly (bf16), fp32
 *    accumulate; the intermediate h is rounded to bf16. Needs T <= 64.
 *  MOE_ACT_FP8_G128_POW2: token rows and h are quantized to e4m3 with one
 *    power-of-two scale per (row, 128 consecutive K elements), the smallest
 *    2^s with max|v| <= 448 * 2^s; FP8 matrix cores, fp32 accumulate. */
enum { MOE_ACT_BF16 = 0, MOE_ACT_FP8_G128_POW2 = 1 };

int         moe_abi_version(void);
const char* moe_strerror(int status);
int         moe_last_hip_error(void);

/* ---------------------------------------------------------------- route
 * [PW] "what was released" / "technically interesting points": a router
 * sends each token to a few experts. Per token t: experts with mask[e] == 0
 * count as -inf; the k chosen are the first k in the order (logit desc,
 * expert id asc), with -0.0 == +0.0; weights are the softmax over the k
 * chosen logits (they sum to 1), computed in fp32.
 *  d_logits  f32 [T, E] row-major.
 *  d_mask    u8 [E] or NULL (all experts allowed).
 *  d_topk_ids i32 [T, k], best first; d_topk_w f32 [T, k].
 *  d_err     i32 [1]: +1 per token with fewer than k allowed experts; such a
 *            token's missing entries get id -1 and weight 0.
 * Limits: 1 <= T, 1 <= k <= min(E, 32), E <= 1024. */
int moe_route(const float* d_logits, const uint8_t* d_mask, int T, int E, int k,
              int32_t* d_topk_ids, float* d_topk_w, int32_t* d_err, void* stream);

/* Route from the token rows: the router gate first, then moe_route.
 * [PW] "technically interesting points": the router picks each token's
 * experts. d_logits[t][e] = sum_h x[t][h] * W_g[e][h] + bias[e] in fp32:
 * W_g is split exactly into three bf16 parts, so every product is exact and
 * the result differs from the exact logit only by the rounding of the fp32
 * sum (at most gamma_{3H} sum_h |x W| + one rounding of the bias add); the
 * order of that sum is fixed, so results repeat from run to run. The logits
 * are written (the caller keeps them) and then routed exactly as moe_route
 * routes them.
 *  d_x bf16 [T, H]; d_wg f32 [E, H]; d_bias f32 [E] or NULL; d_mask as in
 *  moe_route; d_logits f32 [T, E] (output); the rest as in moe_route.
 * Limits: H a multiple of 128; the rest as in moe_route. */
int moe_route_gemm(const uint16_t* d_x, const float* d_wg, const float* d_bias, const uint8_t* d_mask, int T, int H,
                   int E, int k, float* d_logits, int32_t* d_topk_ids, float* d_topk_w, int32_t* d_err,
                   void* stream);

/* ---------------------------------------------------------------- align
 * [MG] sections 1 and 3: tokens are grouped per expert module so each expert
 * runs one large batch. [VEP] "hierarchical paging of expert weights": each
 * layer keeps a table of which expert sits in which VRAM slot.
 * Pair p = t*k + j. Segments in ascending expert id, pairs inside a segment
 * in ascending p, each segment padded to a multiple of block_m with the
 * sentinel T*k; an expert without pairs has no block.
 *  d_sorted_pair  i32 [capacity]; entries [0, n_padded) are defined.
 *  d_block_slot   i32 [capacity / block_m]; entry b is slot_of_expert[e] of
 *                 the expert owning block b (-1 if not resident).
 *  d_counts i32 [E]; d_seg_offset i32 [E + 1] (padded starts; [E] = n_padded);
 *  d_n_padded i32 [1].
 *  d_err i32 [1]: + number of pairs whose id is outside [0, E) (they are
 *        left out) + number of pairs routed to a non-resident expert.
 * block_m in {16, 32, 64, 128, 256}; E <= 1024; T*k < 2^30.
 * The results are bit-identical from run to run. */
int    moe_align_capacity(int T, int k, int E, int block_m);
size_t moe_align_workspace_bytes(int T, int k, int E, int block_m);
int moe_align(const int32_t* d_topk_ids, int T, int k, int E, int block_m,
              const int32_t* d_slot_of_expert,
              int32_t* d_sorted_pair, int32_t* d_block_slot, int32_t* d_counts,
              int32_t* d_seg_offset, int32_t* d_n_padded, int32_t* d_err,
              void* d_ws, size_t ws_bytes, void* stream);

/* Route and align in one call: the same results as moe_route followed by
 * moe_align on the same stream. d_err is i32[2]: [0] gets moe_route's count,
 * [1] moe_align's (the -1 entries of short tokens count there too). The
 * workspace is moe_align's. */
size_t moe_route_align_workspace_bytes(int T, int k, int E, int block_m);
int moe_route_align(const float* d_logits, const uint8_t* d_mask, int T, int E, int k, int block_m,
                    const int32_t* d_slot_of_expert, int32_t* d_topk_ids, float* d_topk_w,
                    int32_t* d_sorted_pair, int32_t* d_block_slot, int32_t* d_counts,
                    int32_t* d_seg_offset, int32_t* d_n_padded, int32_t* d_err,
                    void* d_ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- slot pool
 * [VEP] "hierarchical paging of expert weights": each MoE layer owns a pool
 * of VRAM slots, one expert per slot; the Table 1 set-up names the fused
 * gate+up tensor w13_weight and the down tensor w2_weight.
 * Slot s starts at d_base + s * slot_bytes. Inside a slot each array starts
 * on a 256-byte boundary, in this order:
 *  FP8 : w13 codes u8[2I][H] | w13 scale f32[2I] | w2 codes u8[H][I] | w2 scale f32[H]
 *  INT4: w13 u8[2I][H/2] | w13 (scale, zero) f16[2I][H/128][2]
 *        | w2 u8[H][I/2] | w2 (scale, zero) f16[H][I/128][2]
 *        element c of a row: low nibble of byte c/2 if c is even, else high.
 *  Dequantized: FP8 W[r][c] = e4m3(q[r][c]) * scale[r];
 *               INT4 W[r][c] = (q[r][c] - zero[r][c/128]) * scale[r][c/128].
 *  INT4 zero points are integers in [0, 15] (stored as fp16): the kernels
 *  form q - zero exactly as a small integer before the matrix instructions
 *  and apply the group scale after them (moe_pool_check finds other zeros).
 *  An INT4 slot keeps 16 spare bytes after w2_sz before its size is rounded
 *  up to 256 (moe_slot_bytes includes them).
 * Rows [0, I) of w13 are the gate projection, rows [I, 2I) the up projection.
 * d_slot_fmt is a device array u8[n_slots] of MOE_FMT_* values.
 * hidden % 128 == 0, inter % 64 == 0 (INT4 slots: inter % 128 == 0). */
typedef struct moe_slot_pool {
    void*          d_base;
    size_t         slot_bytes;   /* multiple of 256, >= moe_slot_bytes of some format; slots
                                    whose format does not fit are unusable (not resident) */
    int            n_slots;
    const uint8_t* d_slot_fmt;
    int            hidden;
    int            inter;
} moe_slot_pool;

size_t moe_slot_bytes(int hidden, int inter, int fmt);
/* byte offset of array `part` (0..3 in the order above) inside a slot */
size_t moe_slot_part_offset(int hidden, int inter, int fmt, int part);

/* ---------------------------------------------------------------- expert FFN
 * [VEP] Table 1 set-up and "hierarchical paging" section: the expert's w13
 * and w2 are read from its slot; [PW] "what was released": the layer output
 * mixes the chosen experts' outputs. For every pair p = t*k + j listed in
 * block b (slot s = block_slot[b]; skipped, adding zero, when s is not
 * usable: negative, >= n_slots, or tagged with a format that is not FP8 or
 * int4 or does not fit slot_bytes):
 *    gu = W13[s] a_t, h = silu(gu[0:I]) * gu[I:2I], y = W2[s] h,
 *    out[t] = sum_j topk_w[t][j] * y_(t,j), accumulated in fp32, then bf16.
 * a_t is token row t of x in the precision act_mode selects.
 *  d_x bf16 [T, H]; d_topk_w f32 [T, k]; d_sorted_pair, d_block_slot,
 *  d_n_padded as written by moe_align with the same block_m and E.
 *  d_out bf16 [T, H], fully overwritten (rows of tokens with no resident
 *  expert are zero).
 * block_m: 16, 32 or 64 with MOE_ACT_BF16; 64 or 128 with
 * MOE_ACT_FP8_G128_POW2. The workspace holds moe_ffn_workspace_bytes bytes. */
size_t moe_ffn_workspace_bytes(int T, int k, int E, int hidden, int inter, int block_m, int act_mode);
int moe_expert_ffn(const moe_slot_pool* pool, const uint16_t* d_x, int T, int k, int E,
                   const float* d_topk_w, const int32_t* d_sorted_pair,
                   const int32_t* d_block_slot, const int32_t* d_n_padded,
                   int block_m, int act_mode, uint16_t* d_out,
                   void* d_ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- resident-first passes
 * [EP] "hierarchical paging of expert weights": an expert missing from VRAM
 * is copied in from its host-RAM slot; [MG] section 3: host-to-GPU copies
 * overlap GPU compute. A block whose block_slot entry is MOE_SLOT_DEFERRED
 * is left untouched by moe_expert_ffn_pass: its pairs' rows in the
 * workspace keep their contents (moe_align copies the marker from
 * slot_of_expert and does not count it as an error). moe_expert_ffn_pass is
 * moe_expert_ffn with that rule, and with the combine into d_out run only
 * when last_pass != 0. Two calls on the same stream with the same workspace
 * and sorted pairs, the first deferring the blocks of experts whose slots are
 * still being filled and the second deferring every other block (last_pass =
 * 1), write exactly what one moe_expert_ffn call over the filled pool writes:
 * each pair's row is computed once, by the same kernels. Workspace
 * poisoning (moe_debug_poison) does not apply to these calls. */
#define MOE_SLOT_DEFERRED (-2)
int moe_expert_ffn_pass(const moe_slot_pool* pool, const uint16_t* d_x, int T, int k, int E,
                        const float* d_topk_w, const int32_t* d_sorted_pair, const int32_t* d_block_slot,
                        const int32_t* d_n_padded, int block_m, int act_mode, int last_pass, uint16_t* d_out,
                        void* d_ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- slot-miss path
 * [EP] "hierarchical paging of expert weights": every MoE layer owns its
 * VRAM slots, one expert per slot, managed LRU; an expert that is needed and
 * not in VRAM is copied in from its host-RAM slot. [MG] section 3: the copies
 * run alongside GPU compute (see moe_expert_ffn_pass).
 * moe_pager_create: n_layers layers of E experts and n_slots VRAM slots each,
 * all empty; NULL on bad sizes. moe_pager_plan (host only): for the experts
 * `needed` (host ids; duplicates and ids outside [0, E) ignored) of one step
 * of layer `layer`, a resident expert is a hit; each miss, in ascending
 * expert id, takes the lowest free slot, else the slot of the resident expert
 * not needed by this step that was used least recently (ties to the lower
 * id); then every needed expert counts as used by this step. Writes the
 * layer's table after the step (slot_of_expert, host i32 [E], -1 = not
 * resident) and the fills (fill_expert, fill_slot: host i32 [>= n_slots],
 * *n_fill entries). MOE_EINVAL when the step needs more distinct experts than
 * there are slots (the caller then uses a working buffer that holds them
 * all). moe_pager_stats: hits and misses so far of one layer (-1: all).
 * moe_pager_fill: for each fill i, copies h_bank_stride bytes of host row
 * fill_src[i] of h_bank (page-locked host memory, rows of h_bank_stride <=
 * slot_bytes bytes) into slot fill_slot[i] of the pool, and the row's format
 * tag h_bank_fmt[fill_src[i]] (page-locked) into d_slot_fmt[fill_slot[i]],
 * asynchronously on copy_stream. The caller orders the copies before the
 * kernels that read those slots (an event), and mirrors the plan's table to
 * its device slot table. */
typedef struct moe_pager moe_pager;
moe_pager* moe_pager_create(int n_layers, int E, int n_slots);
void moe_pager_destroy(moe_pager* pager);
int moe_pager_plan(moe_pager* pager, int layer, const int32_t* needed, int n_needed, int32_t* slot_of_expert,
                   int32_t* fill_expert, int32_t* fill_slot, int* n_fill);
int moe_pager_stats(const moe_pager* pager, int layer, long long* hits, long long* misses);
int moe_pager_fill(const moe_slot_pool* pool, const void* h_bank, size_t h_bank_stride, const uint8_t* h_bank_fmt,
                   const int32_t* fill_src, const int32_t* fill_slot, int n_fill, void* copy_stream);

/* ---------------------------------------------------------------- compressed host tier
 * [EP] weight-compression section: FP8 exponents are skewed, so the exponent
 * bits of each row of an expert's matrices are Huffman-coded in host RAM and
 * expanded on the GPU right after the copy into VRAM.
 * Packed slot (every part on a 16-byte boundary): eight u32 (0x38504D46,
 * hidden, inter, offset and size of packed w13, offset and size of packed
 * w2, total size), packed w13 [2I rows x H], w13 row scales f32 [2I], packed
 * w2 [H rows x I], w2 row scales f32 [H]. Packed matrix of R rows x C
 * values (C a multiple of 256): code lengths u8 [R][8] (symbol 2i in the low
 * nibble of byte i), chunk start bits u32 [R][C/256] (bit offsets into the
 * matrix stream), sign|mantissa nibbles u8 [R][C/2] (value c in the low
 * nibble of byte c/2 when c is even), the exponent stream (least significant
 * bit of each byte first), 8 zero bytes. An e4m3 byte is sign | exponent (4
 * bits) | mantissa (3); the exponent is coded. Each row's code is canonical
 * (symbols by (length, symbol) take consecutive codes, written first bit
 * first) with Huffman lengths from the row's exponent counts (merge the two
 * lightest nodes, ties to the node holding the lower symbol; one symbol
 * present: length 1); while a length exceeds 8 the counts of the present
 * symbols are raised by floor(total * 2^k / 256) + 1, k = 0, 1, ... hidden
 * and inter must be multiples of 256.
 * moe_fp8_pack (host only): packs the FP8 slot at h_fp8_slot into h_out
 * (capacity cap >= moe_fp8_pack_bound); returns the packed size (0 = bad
 * arguments). moe_fp8_unpack: expands the packed slot at d_packed (device)
 * into FP8 slot dst_slot and sets its tag to MOE_FMT_FP8_E4M3_ROW; a header
 * that does not match the pool writes nothing and adds 1 to d_err (may be
 * NULL). moe_pager_fill_packed: moe_pager_fill from a host bank of packed
 * slots (row r at h_packed + h_offsets[r], h_sizes[r] bytes, page-locked):
 * each fill is copied into the device staging buffer (the fills' sizes, each
 * rounded up to 16, must fit staging_bytes) and expanded into its slot, all
 * on copy_stream. */
size_t moe_fp8_pack_bound(int hidden, int inter);
size_t moe_fp8_pack(const uint8_t* h_fp8_slot, int hidden, int inter, uint8_t* h_out, size_t cap);
int moe_fp8_unpack(const moe_slot_pool* pool, const uint8_t* d_packed, int dst_slot, int32_t* d_err, void* stream);
int moe_pager_fill_packed(const moe_slot_pool* pool, const uint8_t* h_packed, const uint64_t* h_offsets,
                          const uint64_t* h_sizes, const int32_t* fill_src, const int32_t* fill_slot, int n_fill,
                          uint8_t* d_staging, size_t staging_bytes, int32_t* d_err, void* copy_stream);

/* ---------------------------------------------------------------- whole layer
 * The three steps above in one call: the results of moe_route_align followed
 * by moe_expert_ffn on the same stream, every output written as those calls
 * write it (d_err is i32[2] as in moe_route_align; counts are added).
 * [MG] sections 1 and 3 and [VEP] "hierarchical paging of expert weights"
 * define the sort; [PW] "what was released" the routing and the mixing.
 * Decode-sized layers (T <= 64, T*k <= 512, block_m 16, MOE_ACT_BF16,
 * hidden <= 2048) take fewer launches: every workgroup of the gate/up kernel
 * sorts the pairs in its own LDS instead of waiting for an align launch, and
 * for T <= 16 also routes the tokens itself; other shapes run the separate
 * calls' kernels. The slot table is checked against the pool: an entry that
 * is not usable (>= n_slots, or a slot whose tag is not a usable format)
 * counts like -1 (d_block_slot gets -1, its pairs add zero and count in
 * d_err[1]). The workspace holds moe_layer_workspace_bytes bytes (0 =
 * invalid arguments). Errors: MOE_EINVAL for the arguments any of the three
 * calls rejects. */
size_t moe_layer_workspace_bytes(int T, int k, int E, int hidden, int inter, int block_m, int act_mode);
int moe_layer(const moe_slot_pool* pool, const float* d_logits, const uint8_t* d_mask, const uint16_t* d_x,
              int T, int E, int k, int block_m, int act_mode, const int32_t* d_slot_of_expert,
              int32_t* d_topk_ids, float* d_topk_w, int32_t* d_sorted_pair, int32_t* d_block_slot,
              int32_t* d_counts, int32_t* d_seg_offset, int32_t* d_n_padded, int32_t* d_err,
              uint16_t* d_out, void* d_ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------- activation quantize
 * The activation step of MOE_ACT_FP8_G128_POW2 on its own (the FP8 matrix
 * cores of the grouped contraction need FP8 operands; MOE-GEN explainer,
 * aibr.jp, section 3: per-expert batches are dense contractions). For every
 * row r and group g of 128 consecutive columns: s = the smallest integer with
 * max|x[r][128g..128g+127]| <= 448 * 2^s (s = 0 for an all-zero group),
 * clamped to [-127, 127]; d_codes[r][c] = e4m3 code of x[r][c] / 2^s,
 * rounded to nearest even (x / 2^s is exact); d_exps[r][g] = s + 127 (the
 * E8M0 byte the scaled matrix instruction takes).
 *  d_x bf16 [rows, cols]; d_codes u8 [rows, cols]; d_exps u8 [rows, cols/128].
 * cols must be a positive multiple of 128. */
int moe_quant_act(const uint16_t* d_x, int rows, int cols, uint8_t* d_codes, uint8_t* d_exps, void* stream);

/* ---------------------------------------------------------------- pool check
 * [VEP] "hierarchical paging of expert weights": slots are refilled while
 * the model runs. Every FFN call treats a slot as not resident (its pairs add
 * zero) when its index is outside [0, n_slots), its tag is neither format, or
 * its format's layout does not fit slot_bytes; moe_layer also counts such
 * pairs in d_err[1] and writes -1 for their blocks in d_block_slot.
 * moe_pool_check reports, for every slot, whether it is usable and why not:
 * d_status u8 [n_slots] (may be NULL): 0 usable, 1 the tag is not a format,
 * 2 the format does not fit the stride, 3 an int4 group whose zero point is
 * not an integer in [0, 15] or whose scale is not finite (the kernels form
 * q - zero exactly only for such zero points), 4 an FP8 row scale that is
 * not finite. d_err i32 [1] gets +1 per slot with a nonzero status. */
int moe_pool_check(const moe_slot_pool* pool, int32_t* d_err, uint8_t* d_status, void* stream);

/* ---------------------------------------------------------------- bit width
 * [PW] "technically interesting points": each expert is held at a bit width
 * chosen by how much it matters, switched while the model serves.
 * moe_bitwidth_plan (host arrays, no GPU): fmt_out[e] = MOE_FMT_INT4_G128 for
 * the n_int4 experts with the fewest routed pairs (counts as moe_align
 * writes them; ties to the lower expert id), MOE_FMT_FP8_E4M3_ROW otherwise.
 * moe_requant_slot: the expert in FP8 slot src_slot is requantized into slot
 * dst_slot of the same pool in int4-g128, and d_slot_fmt[dst_slot] is set to
 * MOE_FMT_INT4_G128 (the source slot is left as it is). Per row and group of
 * 128 K values w = e4m3(code) * row_scale (fp32): s = fp16((max - min) / 15)
 * (1 when 0), zero = clip(rint(-min / s), 0, 15), q = clip(rint(w / s) +
 * zero, 0, 15), every step in fp32 with IEEE rounding (ties to even), so the
 * bytes written are fully determined. If src_slot is not a usable FP8 slot
 * nothing is written and d_err (i32 [1], may be NULL) gets +1. Both formats
 * must fit slot_bytes; src_slot != dst_slot. The caller points the expert's
 * slot-table entry at dst_slot when it wants the int4 copy used. */
int moe_bitwidth_plan(const int32_t* counts, int E, int n_int4, uint8_t* fmt_out);
int moe_requant_slot(const moe_slot_pool* pool, int src_slot, int dst_slot, int32_t* d_err, void* stream);

/* ---------------------------------------------------------------- debug
 * moe_debug_poison(1): every later FFN call (moe_expert_ffn, moe_layer)
 * first fills the data regions of its workspace (activation codes, h rows,
 * weighted pair rows) with all-ones bytes, NaN in every float format used,
 * so a read of workspace data the call did not write first shows up as NaN
 * in d_out. Outputs are unchanged when nothing reads unwritten data. A
 * debugging aid (one extra fill per call); moe_debug_poison(0) turns it off.
 * Process-wide. */
int moe_debug_poison(int on);

/* ---------------------------------------------------------------- whole layer, no allocation
 * For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, hosts that forbid
 * allocation): moe_layer with the same arguments and results, minus d_ws and
 * ws_bytes. Its workspace is a fixed array inside the library, one per GPU,
 * of MOE_NOALLOC_SCRATCH_BYTES bytes, held until the process ends; the call
 * allocates nothing. Layers whose moe_layer_workspace_bytes exceeds that
 * size are refused with MOE_ESCRATCH (every decode-sized layer fits: T <= 64
 * tokens with 16-pair blocks and bf16 activations need at most 16 MiB at
 * hidden 2048, inter 768, 1024 experts). All calls on one GPU share the array:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * on it and must be serialised by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_layer_noalloc(const moe_slot_pool* pool, const float* d_logits, const uint8_t* d_mask,
                      const uint16_t* d_x, int T, int E, int k, int block_m, int act_mode,
                      const int32_t* d_slot_of_expert, int32_t* d_topk_ids, float* d_topk_w,
                      int32_t* d_sorted_pair, int32_t* d_block_slot, int32_t* d_counts,
                      int32_t* d_seg_offset, int32_t* d_n_padded, int32_t* d_err, uint16_t* d_out,
                      void* stream);

/* ---------------------------------------------------------------- dequant
 * [PW] "technically interesting points": per-expert bit width. Writes the
 * dequantized matrices of slot `slot` in fp32: d_w13 [2I][H], d_w2 [H][I]
 * (either may be NULL). An unusable slot (see moe_pool_check, statuses 1
 * and 2) yields NaN matrices. */
int moe_dequant_slot(const moe_slot_pool* pool, int slot, float* d_w13, float* d_w2, void* stream);

/* ---------------------------------------------------------------- tracing
 * Launch tracing for measurement (the MOE-GEN explainer, aibr.jp: its
 * dialogue names throughput and GPU utilisation among the figures to watch).
 * moe_profile_enable(1) clears old records and makes every later kernel
 * launch of the library carry a start and a stop HIP event that the dispatch
 * itself stamps, so a pair spans exactly that kernel's execution (not while
 * a stream is being captured); moe_profile_enable(0) stops and frees the
 * events. moe_profile_read() waits for the recorded events of kernel
 * `kernel` (0 <= kernel < moe_profile_kernels(); names from
 * moe_profile_kernel_name) and returns the launch count and the summed
 * milliseconds. Not thread-safe. */
int         moe_profile_enable(int on);
int         moe_profile_kernels(void);
const char* moe_profile_kernel_name(int kernel);
int         moe_profile_read(int kernel, int* launches, double* total_ms);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
