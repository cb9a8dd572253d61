/*
 * moe_routed.h -- C ABI of libmoe_routed: the routed-expert MoE forward on
 * AMD Instinct MI355X (gfx950, CDNA4), one GPU.
 *
 * The forward computes, for every token t with top-k expert ids e_k and
 * routing weights w_k,
 *
 *     y[t] = sum_k w_k * Down_{e_k}( SiLU(Gate_{e_k} x_t) * Up_{e_k} x_t )
 *
 * in three steps, each a call of this library:
 *   0. moe_gate             -- (in front of the path) router logits, top-k
 *                              ids and routing weights on the device;
 *   1. moe_dispatch         -- expert-sorted dispatch tables;
 *   2. moe_expert_gate_up   -- grouped GEMM over the stacked gate/up weights
 *                              with SiLU(gate)*up fused in the epilogue,
 *      moe_expert_down      -- grouped GEMM over the stacked down weights;
 *   3. moe_reduce_fused     -- top-k weighted fp32 reduce back to token order.
 * moe_routed_forward runs step 2 and step 3 back to back. The _weighted
 * variants of the down GEMM and of the forward apply the routing weight in
 * the down GEMM's epilogue instead, and combine with an unweighted reduce.
 *
 * Sources (page title, section):
 *   [A] "tilelang baseline" MoE walkthrough (devpress.csdn.net, tilelang-metax
 *       race): section "forward" (sorting, counts, offsets, padded offsets,
 *       block->expert table), sections "stage-1 gate+up" and "stage-2 down".
 *   [B] TileLang tutorial ch.18 "End-to-end II", skeletons.py,
 *       moe_routed_kernel: the dispatch contract (the kernel takes its
 *       tables from the caller and recovers its rows from them).
 *   [C] TileOPs-Metax PR #55 "moe_reduce_fused": section 1 (design),
 *       section 2 (reference semantics and error cases).
 *
 * Conventions for every call:
 *   - Every array argument is a DEVICE pointer owned by the caller; the
 *     library never allocates or frees memory and keeps no state other than
 *     a thread-local error message.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream). Nothing synchronises with the host. A kernel fault surfaces at
 *     the caller's next synchronisation.
 *   - All argument validation happens on the host before any launch; a call
 *     that returns an error has launched nothing. moe_last_error() then holds
 *     a message naming the argument.
 *   - Row-major layouts throughout. 16-bit tensors (fp16, bf16) hold IEEE
 *     binary16 / bfloat16 bit patterns. Accumulation is fp32; 16-bit results
 *     are rounded to nearest, ties to even.
 *   - Sizes: T tokens, K = top_k slots per token, E experts, H = d_hidden,
 *     D = d_expert, P = T*K routed pairs.
 */
#ifndef MOE_ROUTED_H
#define MOE_ROUTED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL                      */
  MOE_ERR_SHAPE = 2,       /* a size is out of range or not divisible         */
  MOE_ERR_DTYPE = 3,       /* a dtype code is not supported by this call      */
  MOE_ERR_UNSUPPORTED = 4, /* e.g. block_m not in {16, 32, 64, 128, 256}      */
  MOE_ERR_WORKSPACE = 5,   /* the caller's buffer is too small                */
  MOE_ERR_HIP = 6          /* a launch failed (message from the HIP runtime)  */
} moe_status;

/* Storage types. MOE_FP8_E4M3 is OCP FP8 E4M3 ("fn": no infinities, max
 * 448), accepted by the reduce only; casts to it round to nearest even and
 * saturate to +-448. */
typedef enum moe_dtype { MOE_F16 = 0, MOE_BF16 = 1, MOE_F32 = 2, MOE_FP8_E4M3 = 3 } moe_dtype;

/*
 * Dispatch tables ([A] "forward" steps 2-5, [B] dispatch contract).
 * moe_tables_bind() fills this struct with views into ONE caller-allocated
 * device buffer; moe_dispatch() fills the buffer. For a sorted row i
 * (0 <= i < n_valid, rows grouped by expert in ascending expert order and,
 * inside a group, in ascending flat slot order p = t*K + k):
 *   group_sizes[e]          rows routed to expert e                      [E]
 *   group_offsets[e]        exclusive prefix sum of group_sizes          [E]
 *   group_padded_offsets[e] 0 for e = 0, else
 *                           padded[e-1] + ceil((group_sizes[e-1]+1)/block_m)*block_m
 *                           (every expert owns >= 1 block; a group whose size
 *                           is a multiple of block_m gets one extra block)   [E]
 *   block_expert[b]         the last expert e with padded[e] <= b*block_m;
 *                           blocks past the last group belong to E-1
 *                           and hold no rows                       [num_blocks]
 *   sorted_pair[i]          the flat slot p of sorted row i             [P]
 *   sorted_token[i]         p / K                                        [P]
 *   sorted_weight[i]        topk_weights[p] (fp32, copied bit-exactly)   [P]
 *   token_topk_to_pos[p]    the sorted row of slot p, -1 if masked       [P]
 *   topk_weights[p]         fp32 copy of the routing weights, token order [P]
 *   status[0]               0, or 1 if an id >= E was seen (it is then
 *                           treated as a masked slot)                    [1]
 *   active_blocks[j]        the blocks that hold rows, in ascending order:
 *                           expert e contributes blocks padded[e]/block_m
 *                           + 0 .. ceil(group_sizes[e]/block_m) - 1
 *                           (a scheduling list for the GEMMs) [num_blocks]
 *   active_count[0]         the number of entries of active_blocks       [1]
 * Entries i >= n_valid of the sorted_* arrays are unspecified. A slot with a
 * negative id is masked: it is not counted and never read. The scan scratch
 * (chunk_counts, chunk_flags, pair_rank) is internal. moe_dispatch writes
 * every table entry it defines on each call (no memset is needed, so the
 * call may be captured into a HIP graph).
 */
typedef struct moe_tables {
  int32_t T, K, E, block_m;
  int32_t num_blocks; /* ceil(T*K / block_m) + E                          */
  int32_t num_chunks; /* ceil(T*K / 1024): dispatch scan chunks            */
  int32_t *group_sizes, *group_offsets, *group_padded_offsets;
  int32_t *block_expert;
  int32_t *sorted_pair, *sorted_token;
  float *sorted_weight;
  int32_t *token_topk_to_pos;
  float *topk_weights;
  int32_t *status;
  int32_t *active_blocks;
  int32_t *active_count;
  int32_t *chunk_counts; /* [num_chunks * E] */
  int32_t *chunk_flags;  /* [num_chunks]     */
  int32_t *pair_rank;    /* [P]              */
} moe_tables;

/* Step 0 (in front of the path): the router gate. The routed-MoE workload
 * recipes define it: router weights Wr [E, H] in fp32, fp32 softmax of the
 * logits x . Wr^T, the top-k experts by score with ties to the lower expert
 * index, routing weights = the selected scores, renormalised to sum to 1
 * where asked; the skewed workload adds a per-expert bias to the logits.
 *   x             [T, H] of dtype (MOE_F16, MOE_BF16 or MOE_F32);
 *   w_router      fp32 [E, H];
 *   bias          fp32 [E] added to every token's logits, or NULL;
 *   logits        fp32 [T, E] output: logits[t, e] = (one fp32 fused
 *                 multiply-add chain over h = 0..H-1 ascending of
 *                 x[t, h] * w_router[e, h]) + bias[e] -- reproducible bit
 *                 for bit under that definition;
 *   topk_ids      int32 [T, K] output: the K largest logits of each token
 *                 in descending order, ties to the lower index (ranking by
 *                 logit is ranking by score: the softmax is increasing);
 *   topk_weights  fp32 [T, K] output: softmax(logits[t])[topk_ids[t, k]],
 *                 divided by their sum over k when renorm != 0.
 * The outputs feed moe_dispatch directly. Inputs must be finite.
 * Requires H % 64 == 0, 1 <= E <= 1024, 1 <= K <= min(E, 64), T >= 0.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_HIP. */
moe_status moe_gate(const void* x, const float* w_router, const float* bias, int T, int H, int E,
                    int K, int renorm, int dtype, float* logits, int32_t* topk_ids,
                    float* topk_weights, void* stream);

/* Human-readable name of a status code; never NULL. */
const char* moe_status_string(int status);

/* Message of the last failing call on this thread ("" if none). */
const char* moe_last_error(void);

/* Bytes of device memory the tables need (0 if the sizes are invalid:
 * T >= 1, 1 <= K <= 64, 1 <= E <= 1024, block_m in {16,32,64,128,256},
 * T*K < 2^31). */
size_t moe_tables_bytes(int T, int K, int E, int block_m);

/* Carve `tables` out of `buffer` (device memory of at least `bytes` bytes,
 * 256-byte aligned). Host-only: touches no device memory.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_UNSUPPORTED (block_m),
 * MOE_ERR_WORKSPACE (bytes < moe_tables_bytes). */
moe_status moe_tables_bind(moe_tables* tables, void* buffer, size_t bytes, int T, int K,
                           int E, int block_m);

/* Step 1: build the dispatch tables from the router output ([A] "forward";
 * [B] dispatch contract; the inverse map token_topk_to_pos is the input of
 * [C]'s reduce).
 *   topk_ids      int32 [T, K]; values in [0, E), or negative = masked slot.
 *   topk_weights  fp32 [T, K]; NULL means every weight is 1.
 * Deterministic: the permutation is stable in p (a counting sort built from
 * wavefront ballots and prefix scans; no atomics decide any position).
 * Errors: MOE_ERR_NULL (tables, topk_ids, or unbound tables), MOE_ERR_HIP. */
moe_status moe_dispatch(const int32_t* topk_ids, const float* topk_weights,
                        moe_tables* tables, void* stream);

/* Step 2a: grouped gate/up GEMM with fused SiLU(gate)*up ([A] "stage-1
 * gate+up"; [B] moe_routed_kernel, first kernel).
 *   x       [T, H] dtype;  w_gate, w_up [E, D, H] dtype (stacked, one [D, H]
 *           matrix per expert, so both GEMMs contract over contiguous rows).
 *   h       [P, D] dtype output, row i = sorted row i:
 *           h[i, j] = R( SiLU(g) * u ),  g = x[sorted_token[i]] . w_gate[e, j],
 *           u = x[sorted_token[i]] . w_up[e, j], e the expert of row i,
 *           SiLU(g) = g / (1 + exp(-g)), fp32 accumulation, R = rounding to
 *           dtype. Rows >= n_valid are not written.
 *   dtype   MOE_BF16 or MOE_F16 (MFMA kernels), or MOE_F32 (the debug path:
 *           fp32 inputs and intermediates, no rounding, vector-ALU kernel
 *           with each dot product one fmaf chain in ascending order).
 * Requires H % 256 == 0 and D % 128 == 0.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_HIP. */
moe_status moe_expert_gate_up(const void* x, const void* w_gate, const void* w_up,
                              const moe_tables* tables, int H, int D, int dtype, void* h,
                              void* stream);

/* Step 2b: grouped down GEMM ([A] "stage-2 down"; [B] moe_routed_kernel,
 * second kernel), WITHOUT the routing weight (it is applied once, in the
 * reduce, as [C] does):
 *   h           [P, D] dtype (the output of moe_expert_gate_up);
 *   w_down      [E, H, D] dtype;
 *   expert_out  [P, H] dtype output: expert_out[i, c] = R( h[i] . w_down[e, c] ).
 * Same requirements and errors as moe_expert_gate_up. */
moe_status moe_expert_down(const void* h, const void* w_down, const moe_tables* tables, int H,
                           int D, int dtype, void* expert_out, void* stream);

/* Step 2b with the routing weight in the epilogue ([B] moe_routed_kernel,
 * second kernel: each output row is multiplied by its row weight before it
 * is written, so the combine needs no weights):
 *   expert_out[i, c] = R( sorted_weight[i] * (h[i] . w_down[e, c]) ),
 * the product taken in fp32 on the accumulated dot product, then rounded
 * once to dtype. sorted_weight comes from the tables (moe_dispatch's copy
 * of topk_weights; all ones if it was given NULL). Feed the result to
 * moe_reduce_fused with topk_weights = NULL.
 * Same arguments, requirements and errors as moe_expert_down. */
moe_status moe_expert_down_weighted(const void* h, const void* w_down, const moe_tables* tables,
                                    int H, int D, int dtype, void* expert_out, void* stream);

/* Workspace of moe_routed_forward: h [P, D] at offset 0, then expert_out
 * [P, H] at the next 256-byte boundary (both of dtype). 0 if invalid. */
size_t moe_forward_workspace_bytes(int T, int K, int H, int D, int dtype);

/* Byte offset of expert_out inside that workspace. */
size_t moe_forward_workspace_expert_out_offset(int T, int K, int H, int D, int dtype);

/* Steps 2-3: y [T, H] dtype = moe_reduce_fused(moe_expert_down(moe_expert_gate_up(x)),
 * tables->token_topk_to_pos, tables->topk_weights). The intermediates stay
 * in `workspace` (layout above) and may be read back by the caller.
 * Errors: as the three steps, plus MOE_ERR_WORKSPACE. */
moe_status moe_routed_forward(const void* x, const void* w_gate, const void* w_up,
                              const void* w_down, const moe_tables* tables, int H, int D,
                              int dtype, void* workspace, size_t workspace_bytes, void* y,
                              void* stream);

/* Steps 2a + 2b fused for decode-sized row blocks ([A] "stage-2 down",
 * which notes that the two stages can be fused so that h is never stored):
 * one workgroup per row block computes the block's h (at most 32 rows x D)
 * into on-chip memory (LDS), then the block's expert_out rows from it.
 *   expert_out [P, H] dtype output, bit-identical to
 *              moe_expert_down(moe_expert_gate_up(x)) (same rounding of h,
 *              same summation order).
 * Requires tables built with block_m <= 32, D <= MOE_FUSED_MAX_D_EXPERT
 * (h of a block must fit in LDS), dtype MOE_BF16 or MOE_F16, and the
 * requirements of moe_expert_gate_up.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_UNSUPPORTED
 * (block_m > 32 or D > MOE_FUSED_MAX_D_EXPERT), MOE_ERR_HIP. */
#define MOE_FUSED_MAX_D_EXPERT 2048
moe_status moe_expert_fused(const void* x, const void* w_gate, const void* w_up,
                            const void* w_down, const moe_tables* tables, int H, int D,
                            int dtype, void* expert_out, void* stream);

/* Workspace of moe_routed_forward_fused: expert_out [P, H] dtype only (no h).
 * 0 if the sizes are invalid. */
size_t moe_fused_workspace_bytes(int T, int K, int H, int dtype);

/* Steps 2-3 with the fused expert kernel: y [T, H] dtype =
 * moe_reduce_fused(moe_expert_fused(x), token_topk_to_pos, topk_weights),
 * bit-identical to moe_routed_forward. `workspace` holds expert_out
 * (moe_fused_workspace_bytes, 256-byte aligned).
 * Errors: as moe_expert_fused and moe_reduce_fused, plus MOE_ERR_WORKSPACE. */
moe_status moe_routed_forward_fused(const void* x, const void* w_gate, const void* w_up,
                                    const void* w_down, const moe_tables* tables, int H, int D,
                                    int dtype, void* workspace, size_t workspace_bytes, void* y,
                                    void* stream);

/* Steps 2-3 without allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): moe_routed_forward with its workspace (h, then
 * expert_out, the layout above) taken from a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends (80 MiB: enough for T*K = 4096 routed pairs at
 * d_hidden 7168, d_expert 2048 in a 16-bit dtype). The caller still passes
 * every input and y. Same result, requirements and errors as
 * moe_routed_forward, plus MOE_ERR_WORKSPACE when
 * moe_forward_workspace_bytes(T, K, H, D, dtype) exceeds the array (nothing
 * is launched then). No call of it allocates memory. Every call on one GPU
 * shares that GPU's array, which keeps the last call's contents: calls
 * that overlap on one GPU (on two streams or from two threads) race. */
#define MOE_NOALLOC_SCRATCH_BYTES (80u << 20)
moe_status moe_routed_forward_noalloc(const void* x, const void* w_gate, const void* w_up,
                                      const void* w_down, const moe_tables* tables, int H, int D,
                                      int dtype, void* y, void* stream);

/* Steps 2-3 with the weighted down epilogue ([B] moe_routed_kernel):
 *   y [T, H] dtype = moe_reduce_fused(moe_expert_down_weighted(
 *                        moe_expert_gate_up(x)), token_topk_to_pos, NULL),
 * i.e. y[t] = R( sum over k ascending with pos[t,k] >= 0 of
 *                R(w[t,k] * (h . w_down)) ) in fp32. The two forms round at
 * different points, so their results may differ in the last bits; both are
 * deterministic. Same workspace (its expert_out then holds weighted rows),
 * requirements and errors as moe_routed_forward. */
moe_status moe_routed_forward_weighted(const void* x, const void* w_gate, const void* w_up,
                                       const void* w_down, const moe_tables* tables, int H,
                                       int D, int dtype, void* workspace,
                                       size_t workspace_bytes, void* y, void* stream);

/* Quantised expert weights (FP8 E4M3 with one fp32 scale per weight row,
 * i.e. per output channel; activations, h, expert_out and y stay in the
 * 16-bit dtype). The pages leave the quantisation scheme open; this one
 * halves the weight bytes the decode layer streams.
 *
 * moe_quantize_fp8_rows: for each of `rows` rows of `cols` values of dtype
 * (MOE_F16, MOE_BF16, MOE_F32) in w, writes
 *   scales[r] = max_k |w[r,k]| / 448 (1 for an all-zero row) and
 *   q[r, k]   = E4M3(w[r, k] / scales[r])  (fp32 division, round to nearest
 *               even, saturating at +-448).
 * Stacked weights [E, N, Kd] are E*N rows of Kd. A one-time conversion.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_HIP. */
moe_status moe_quantize_fp8_rows(const void* w, int64_t rows, int cols, int dtype, uint8_t* q,
                                 float* scales, void* stream);

/* moe_expert_gate_up / moe_expert_down with FP8 weights: w_gate, w_up
 * [E, D, H] and w_down [E, H, D] hold E4M3 codes; s_gate, s_up [E, D] and
 * s_down [E, H] the fp32 row scales. Each dot product runs over the decoded
 * codes (exact in the 16-bit dtype), then is multiplied by its row's scale:
 *   g = s_gate[e,j] * (x . Wg8[e,j]),  u = s_up[e,j] * (x . Wu8[e,j]),
 *   h = R(SiLU(g) * u),  expert_out[i,c] = R(s_down[e,c] * (h . Wd8[e,c])).
 * dtype: MOE_F16 or MOE_BF16. Other requirements and errors as the 16-bit
 * calls. moe_routed_forward_w8 runs both and moe_reduce_fused (workspace as
 * moe_routed_forward). */
moe_status moe_expert_gate_up_w8(const void* x, const uint8_t* w_gate, const uint8_t* w_up,
                                 const float* s_gate, const float* s_up, const moe_tables* tables,
                                 int H, int D, int dtype, void* h, void* stream);
moe_status moe_expert_down_w8(const void* h, const uint8_t* w_down, const float* s_down,
                              const moe_tables* tables, int H, int D, int dtype, void* expert_out,
                              void* stream);
moe_status moe_routed_forward_w8(const void* x, const uint8_t* w_gate, const uint8_t* w_up,
                                 const uint8_t* w_down, const float* s_gate, const float* s_up,
                                 const float* s_down, const moe_tables* tables, int H, int D,
                                 int dtype, void* workspace, size_t workspace_bytes, void* y,
                                 void* stream);

/* W4A8 experts ([B] w4a8_dequant_gemm and the module docstring's weight +
 * activation mode: int4 weights packed two per uint8, int8 activations,
 * int32 accumulation; the quantisation scheme is left open by the pages and
 * taken here as symmetric per row).
 * Packed int4 rows: field 2i in bits 0..3 of byte i, field 2i+1 in bits
 * 4..7, each a 4-bit two's complement number in [-8, 7].
 *
 * moe_quantize_int8_rows: per row r of `rows` rows of `cols` values of dtype
 * (MOE_F16, MOE_BF16, MOE_F32): scales[r] = max_k |a[r,k]| / 127 (1 for an
 * all-zero row), q[r,k] = clamp(nearest integer to a[r,k] / scales[r] (fp32
 * division, ties to even), -127, 127). q int8 [rows, cols], scales fp32 [rows].
 *
 * moe_quantize_int4_rows: the same with 7 in place of 127 and codes clamped
 * to [-8, 7], packed: packed uint8 [rows, cols / 2] (cols even).
 * Both: errors MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_HIP. */
moe_status moe_quantize_int8_rows(const void* a, int64_t rows, int cols, int dtype, int8_t* q,
                                  float* scales, void* stream);
moe_status moe_quantize_int4_rows(const void* w, int64_t rows, int cols, int dtype,
                                  uint8_t* packed, float* scales, void* stream);

/* The plain W4A8 GEMM of [B] w4a8_dequant_gemm:
 *   Ct[n, m] = sum_k A[m, k] * B4[n, k]   (exact, int32)
 *   A  int8 [M, K];  B  packed int4 uint8 [N, K/2];  Ct  int32 [N, M]
 *   (written transposed, as in [B]).
 * Requires M >= 1, N % 256 == 0, K % 256 == 0 and K <= 131072 (the kernel
 * accumulates 16 x the products in int32). Ct is overwritten. Errors:
 * MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_HIP. */
moe_status moe_w4a8_gemm(const int8_t* A, const uint8_t* B, int M, int N, int K, int32_t* Ct,
                         void* stream);

/* moe_expert_gate_up / moe_expert_down with W4A8 experts: w_gate, w_up
 * packed int4 [E, D, H/2] and w_down [E, H, D/2] with fp32 row scales
 * s_gate, s_up [E, D], s_down [E, H]; activations int8 with one fp32 scale
 * per row: xq [T, H] with sx [T] (token order; gathered through
 * sorted_token), hq [P, D] with sh [P] (sorted order). With
 * dq(acc, sa, sw) = (float) acc * sa * sw (fp32, left to right):
 *   g = dq(xq[t] . Wg4[e,j], sx[t], s_gate[e,j]),  u likewise,
 *   h[i, j] = R(SiLU(g) * u),
 *   expert_out[i, c] = R(dq(hq[i] . Wd4[e,c], sh[i], s_down[e,c])),
 * dot products exact in int32. dtype (of h / expert_out): MOE_F16 or
 * MOE_BF16. Requires D % 256 == 0 besides the 16-bit calls' rules.
 *
 * moe_routed_forward_w4a8 runs: x -> xq, sx (moe_quantize_int8_rows);
 * gate/up -> h; h -> hq, sh (per sorted row); down -> expert_out;
 * moe_reduce_fused -> y. Its workspace (moe_forward_w4a8_workspace_bytes,
 * 256-byte aligned) holds h, expert_out (as moe_routed_forward's) and then
 * xq, sx, hq, sh. Errors as the 16-bit calls. */
moe_status moe_expert_gate_up_w4a8(const int8_t* xq, const float* sx, const uint8_t* w_gate,
                                   const uint8_t* w_up, const float* s_gate, const float* s_up,
                                   const moe_tables* tables, int H, int D, int dtype, void* h,
                                   void* stream);
moe_status moe_expert_down_w4a8(const int8_t* hq, const float* sh, const uint8_t* w_down,
                                const float* s_down, const moe_tables* tables, int H, int D,
                                int dtype, void* expert_out, void* stream);
size_t moe_forward_w4a8_workspace_bytes(int T, int K, int H, int D, int dtype);
moe_status moe_routed_forward_w4a8(const void* x, const uint8_t* w_gate, const uint8_t* w_up,
                                   const uint8_t* w_down, const float* s_gate, const float* s_up,
                                   const float* s_down, const moe_tables* tables, int H, int D,
                                   int dtype, void* workspace, size_t workspace_bytes, void* y,
                                   void* stream);

/* W8A8 experts ([B] module docstring: the weight + activation mode, both
 * GEMM operands quantised; the scheme is left open by the pages and taken
 * here as E4M3 codes with one fp32 scale per row on both sides): the FP8
 * weights of moe_quantize_fp8_rows (codes [E, D, H] / [E, D, H] / [E, H, D],
 * scales [E, D] / [E, D] / [E, H]) against FP8 activations quantised by the
 * same call: xq [T, H] with sx [T] (token order; gathered through
 * sorted_token) and hq [P, D] with sh [P] (sorted order), both 16-byte
 * aligned. Each dot product is accumulated in fp32 over the exact products
 * of the E4M3 values (by the FP8 MFMA, in its own order), then scaled once:
 *   g = (xq[t] . Wg8[e,j]) * sx[t] * s_gate[e,j]  (fp32, left to right),
 *   u likewise,  h[i, j] = R(SiLU(g) * u),
 *   expert_out[i, c] = R((hq[i] . Wd8[e,c]) * sh[i] * s_down[e,c]).
 * dtype (of h / expert_out): MOE_F16 or MOE_BF16; the 16-bit calls' shape
 * rules. moe_routed_forward_w8a8 runs: x -> xq, sx (moe_quantize_fp8_rows
 * per token); gate/up -> h; h -> hq, sh (per sorted row); down ->
 * expert_out; moe_reduce_fused -> y. Its workspace
 * (moe_forward_w8a8_workspace_bytes, 256-byte aligned): h, expert_out as
 * moe_routed_forward's, then xq, sx, hq, sh. Errors as the 16-bit calls. */
moe_status moe_expert_gate_up_w8a8(const uint8_t* xq, const float* sx, const uint8_t* w_gate,
                                   const uint8_t* w_up, const float* s_gate, const float* s_up,
                                   const moe_tables* tables, int H, int D, int dtype, void* h,
                                   void* stream);
moe_status moe_expert_down_w8a8(const uint8_t* hq, const float* sh, const uint8_t* w_down,
                                const float* s_down, const moe_tables* tables, int H, int D,
                                int dtype, void* expert_out, void* stream);
size_t moe_forward_w8a8_workspace_bytes(int T, int K, int H, int D, int dtype);
moe_status moe_routed_forward_w8a8(const void* x, const uint8_t* w_gate, const uint8_t* w_up,
                                   const uint8_t* w_down, const float* s_gate, const float* s_up,
                                   const float* s_down, const moe_tables* tables, int H, int D,
                                   int dtype, void* workspace, size_t workspace_bytes, void* y,
                                   void* stream);

/* Block-scaled (MX) experts ([B] module docstring: the block-scaled mode,
 * gemm_blockscaled with per-block scale factors of both operands; formats
 * as the OCP Microscaling specification v1.0 defines them): along a row,
 * every block of 32 values shares one E8M0 scale byte e (X = 2^(e-127));
 * elements are FP8 E4M3 (MOE_MX_FP8: one byte each) or FP4 E2M1 (MOE_MX_FP4:
 * two per byte, element 2i in bits 0..3).
 *
 * moe_quantize_mx_rows: per 32-block with amax = max |v|:
 *   e = floor(log2 amax) - emax_elem + 127 (emax_elem 8 for E4M3, 2 for
 *       E2M1; clamped to [0, 254]; 127 for an all-zero block),
 *   element = the grid value nearest to v / X (fp32 division, ties to the
 *       even code, saturating at the largest magnitude).
 *   v [rows, cols] of dtype (MOE_F16, MOE_BF16, MOE_F32), cols % 32 == 0;
 *   codes [rows, cols] (FP8) or [rows, cols/2] (FP4), 16-byte aligned;
 *   scales uint8 [rows, cols/32].
 *
 * moe_expert_gate_up_mx / moe_expert_down_mx: MXFP4 weights w_gate, w_up
 * [E, D, H/2] and w_down [E, H, D/2] with scales [E, D, H/32] / [E, H, D/32]
 * against MXFP8 activations xq [T, H] with xs [T, H/32] (token order) and
 * hq [P, D] with hs [P, D/32] (sorted order); every dot product is
 * sum_k (X_a a_k)(X_w w_k), accumulated in fp32 by the scaled MFMA:
 *   h = R(SiLU(g) * u),  expert_out = R(hq . Wd).
 * dtype (of h / expert_out): MOE_F16 or MOE_BF16; D % 256 == 0 besides the
 * 16-bit calls' rules. moe_routed_forward_mx: x -> MXFP8; gate/up; h ->
 * MXFP8 per sorted row; down; moe_reduce_fused. Workspace
 * (moe_forward_mx_workspace_bytes, 256-byte aligned): h, expert_out as
 * moe_routed_forward's, then xq, xs, hq, hs. Errors as the 16-bit calls. */
#define MOE_MX_FP8 0
#define MOE_MX_FP4 4
moe_status moe_quantize_mx_rows(const void* v, int64_t rows, int cols, int dtype, int fmt,
                                uint8_t* codes, uint8_t* scales, void* stream);
moe_status moe_expert_gate_up_mx(const uint8_t* xq, const uint8_t* xs, const uint8_t* w_gate,
                                 const uint8_t* w_up, const uint8_t* s_gate, const uint8_t* s_up,
                                 const moe_tables* tables, int H, int D, int dtype, void* h,
                                 void* stream);
moe_status moe_expert_down_mx(const uint8_t* hq, const uint8_t* hs, const uint8_t* w_down,
                              const uint8_t* s_down, const moe_tables* tables, int H, int D,
                              int dtype, void* expert_out, void* stream);
size_t moe_forward_mx_workspace_bytes(int T, int K, int H, int D, int dtype);
moe_status moe_routed_forward_mx(const void* x, const uint8_t* w_gate, const uint8_t* w_up,
                                 const uint8_t* w_down, const uint8_t* s_gate, const uint8_t* s_up,
                                 const uint8_t* s_down, const moe_tables* tables, int H, int D,
                                 int dtype, void* workspace, size_t workspace_bytes, void* y,
                                 void* stream);

/* Step 3: top-k weighted reduce back to token order ([C] sections 1-2):
 *   y[t, :] = R_out( sum over k = 0..K-1 ascending with pos[t,k] >= 0 of
 *                    w[t,k] * expert_out[pos[t,k], :] )
 * accumulated in fp32 with fused multiply-add in k order, cast once at the
 * end. Slots with pos < 0 are neither read nor accumulated; a token whose
 * slots are all masked gets zeros.
 *   expert_out         [rows, H] of in_dtype;
 *   token_topk_to_pos  int32 [T, K], each value < rows;
 *   topk_weights       fp32 [T, K], or NULL for all-ones weights;
 *   in_dtype/out_dtype MOE_F16, MOE_BF16, MOE_F32 or MOE_FP8_E4M3;
 *   y                  [T, H] of out_dtype.
 * Requires H % 256 == 0 ([C] section 2 lists H % 256 != 0 as an error case).
 * A position >= rows is a precondition violation; the kernel skips it.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_HIP. */
moe_status moe_reduce_fused(const void* expert_out, int64_t rows,
                            const int32_t* token_topk_to_pos, const float* topk_weights, int T,
                            int K, int H, int in_dtype, int out_dtype, void* y, void* stream);

/* The scaled / FP8 variants of the reduce ([C] section 1: the with_x_sf and
 * with_sf switches and the FP8-output and quantized variants, one kernel):
 *   y[t, :] = R_out( sf[t] * sum over k ascending with pos[t,k] >= 0 of
 *                    (w[t,k] * x_sf[pos[t,k]]) * expert_out[pos[t,k], :] )
 *   x_sf   fp32 [rows]: a scale per expanded row (per routed slot's row), one
 *          multiply per slot; NULL = ones.
 *   sf     fp32 [T]: a scale per token applied to the fp32 sum, one multiply
 *          per output element; NULL = ones.
 *   in_dtype / out_dtype: MOE_F16, MOE_BF16, MOE_F32 or MOE_FP8_E4M3
 *          (e.g. FP8 rows with x_sf in, FP8 out with sf: the quantized form).
 * Same requirements and errors as moe_reduce_fused. */
moe_status moe_reduce_fused_scaled(const void* expert_out, int64_t rows,
                                   const int32_t* token_topk_to_pos, const float* topk_weights,
                                   const float* x_sf, const float* sf, int T, int K, int H,
                                   int in_dtype, int out_dtype, void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTED_H */
