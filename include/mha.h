/*
 * mha.h -- C ABI of the MI355X (gfx950) multi-head scaled dot-product
 * attention forward library, libmha.so.
 *
 * What is computed (the pages' definitions):
 *   Attention(Q, K, V) = softmax(Q K^T / sqrt(d_k)) V over the key axis, with
 *   masked scores replaced by -1e9 after scaling (The Annotated Transformer,
 *   "Attention" section; "Transformer" study notes, attention-mechanism
 *   section).  MultiHead(Xq, Xkv) = Concat(head_1..head_h) W_O^T + b_O with
 *   head_i = Attention(Q_i, K_i, V_i), Q = Xq W_Q^T + b_Q, K = Xkv W_K^T + b_K,
 *   V = Xkv W_V^T + b_V, and head i owning features [i*d_k, (i+1)*d_k)
 *   ("Transformer" study notes, multi-head attention formula, parameter list
 *   and class: four d_model x d_model linear layers, view/transpose split,
 *   transpose/view merge).
 *
 * Masks.  For query i of batch b, key j is allowed when
 *   (valid_lens == NULL || j < valid_lens[b]) && (!causal || j <= i).
 *   valid_lens is the d2l key-padding length, one per batch, shared by every
 *   head (d2l Transformer digest, multi-head attention prerequisites; no
 *   query attends padded keys).  causal is the lower-triangular subsequent
 *   mask that keeps the diagonal ("Transformer" study notes, mask-generation
 *   section, printed 5x5 example).  Both together are combined by AND.
 *   Because the fill REPLACES the score with -1e9, a query whose keys are all
 *   masked (valid_lens[b] <= 0) weights all Lk keys uniformly; for every other
 *   query a masked key contributes exactly zero.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no per-call state, and enqueues its kernels on
 *     `stream` (a hipStream_t; NULL = the null stream).  Calls return as soon
 *     as the work is enqueued; results are ready after the stream syncs.
 *   - Every argument is checked on the host before anything is enqueued; on
 *     any error nothing is written.
 *   - Errors: MHA_EINVAL (null required pointer, negative or inconsistent
 *     sizes, d_model != h * d_k, causal with Lq != Lk, misaligned pointers or
 *     strides, output aliasing an input); MHA_ENOTSUP (d_k or d_v other than
 *     64, an unsupported dtype pair, or sizes past the kernels' 32-bit
 *     offsets: an activation operand of mha_forward / mha_forward_ex /
 *     mha_sublayer_forward with B * L * d_model >= 2^31 elements, a row
 *     stride of sdpa_forward with 128 rows >= 2^31 bytes, or, on the bf16
 *     backward and weights paths, one (batch, head)'s rows spanning >= 2^31
 *     bytes); MHA_EWORKSPACE (workspace too small);
 *     MHA_EHIP (the HIP runtime reported an error when enqueuing).  Faults of
 *     the device itself surface when the caller synchronises the stream.
 *   - dtypes: MHA_F32 computes in fp32 throughout (FMA, no reduced
 *     precision).  MHA_BF16 takes bf16 inputs and weights, multiplies on bf16
 *     MFMA with fp32 accumulation, keeps the softmax state in fp32, and writes
 *     the output as bf16 or fp32 (out_dt).  With MHA_BF16, mha_forward
 *     carries Q (times log2(e)/sqrt(d_k)) and K as bf16 hi + lo pairs
 *     (hi = bf16(x), lo = bf16(x - hi)) whose scores are formed from three
 *     bf16 products (hi.hi + lo.hi + hi.lo), so large logits, such as those
 *     of embeddings scaled by sqrt(d_model), keep near-fp32 accuracy instead
 *     of moving by a bf16 rounding step; V and the merged head output are
 *     rounded to bf16.  Two routes compute this: for short sequences (K and
 *     V re-projected at most 1.5 times over the blocks of 256 queries, at
 *     most 512 keys) each head's Q, K and V are projected inside its
 *     attention kernel and stay on chip; otherwise one GEMM launch writes
 *     the hi + lo projections to the workspace and the attention kernel
 *     reads them.  sdpa_forward's and sdpa_decode's bf16 inputs are
 *     exact bf16 values and use a single product.
 */
#ifndef MHA_H
#define MHA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MHA_F32 = 0, MHA_BF16 = 1 } mha_dtype;

typedef enum {
    MHA_OK = 0,
    MHA_EINVAL = 1,
    MHA_ENOTSUP = 2,
    MHA_EWORKSPACE = 3,
    MHA_EHIP = 4
} mha_status;

/* Element strides of a [batch, head, position, feature] view whose feature
 * axis is contiguous (stride 1).  [B, h, L, d] contiguous is
 * {h*L*d, L*d, d}; the [B, L, h*d] layout of a linear layer's output viewed
 * per head is {L*h*d, d, h*d}. */
typedef struct {
    long long b, h, l;
} mha_strides;

/*
 * sdpa_forward -- scaled dot-product attention on split heads.
 *
 *   q : [B, h, Lq, d_k] per `sq`        k : [B, h, Lk, d_k] per `sk`
 *   v : [B, h, Lk, d_v] per `sv`        o : [B, h, Lq, d_v] per `so` (written)
 *   valid_lens : device int32 [B], or NULL for no padding mask.
 *   causal     : nonzero applies the subsequent mask (requires Lq == Lk).
 *   in_dt      : dtype of q, k, v.  out_dt: dtype of o.  MHA_F32 inputs
 *                require an MHA_F32 output.
 *   Requirements: d_k == d_v == 64; B, h, Lq >= 0; Lk >= 1; pointers 16-byte
 *   aligned; strides multiples of 8 (bf16) or 4 (fp32) elements; o must not
 *   overlap q, k or v.  B == 0 or Lq == 0 is a no-op.
 * The scale is 1/sqrt(d_k) (d_k = the per-head width); it is not a parameter.
 */
mha_status sdpa_forward(mha_dtype in_dt, mha_dtype out_dt,
                        const void* q, mha_strides sq,
                        const void* k, mha_strides sk,
                        const void* v, mha_strides sv,
                        void* o, mha_strides so,
                        int B, int h, int Lq, int Lk, int d_k, int d_v,
                        const int* valid_lens, int causal, void* stream);

/*
 * sdpa_forward_lse -- sdpa_forward that also writes each query's log-sum-exp
 * of its scaled scores, the statistic a training step keeps for the
 * backward pass (the pages train these models: d2l Transformer digest,
 * training; The Annotated Transformer, Part 2).  The softmax of the
 * "Attention" section's attention() normalises by the sum of exp(s_ij) over
 * the allowed keys j (s_ij = q_i . k_j / sqrt(d_k)); lse_i is the natural
 * log of that sum, so the weights are exp(s_ij - lse_i).
 *   lse : device fp32, B*h*Lq elements, 4-byte aligned, element (b, hd, i)
 *         at (b*h + hd)*Lq + i (written); must not overlap q, k, v or o.  A
 *         row with no allowed key (length <= 0) weighs its Lk keys equally
 *         and gets ln(Lk).  NULL is MHA_EINVAL unless B*Lq == 0.
 * Everything else as sdpa_forward; the kernels are sdpa_forward's, which
 * form the statistic in their last step (log2 units, converted here).
 */
mha_status sdpa_forward_lse(mha_dtype in_dt, mha_dtype out_dt,
                            const void* q, mha_strides sq,
                            const void* k, mha_strides sk,
                            const void* v, mha_strides sv,
                            void* o, mha_strides so,
                            int B, int h, int Lq, int Lk, int d_k, int d_v,
                            const int* valid_lens, int causal, float* lse, void* stream);

/*
 * sdpa_decode -- one incremental-decoding step: a single new query per
 * (batch, head) attends to that head's cached keys and values.  At
 * prediction time the pages' decoder concatenates the keys and values of all
 * earlier steps with the current one and attends from the current position
 * (d2l Transformer digest, decoder block state); the result equals
 * sdpa_forward with Lq = 1, Lk = L, valid_lens = lens and causal = 0.
 *
 *   q    : [B, h, d_k] per {sq.b, sq.h} (sq.l unused)
 *   k, v : caches [B, h, L, d_k] per sk, sv (bf16); the current step's key
 *          and value must already be stored at position lens[b] - 1.
 *   lens : device int32 [B] (required): positions 0 .. lens[b]-1 are
 *          attended; values above L count as L, and lens[b] <= 0 weights all
 *          L positions uniformly (the fully masked row).
 *   o    : [B, h, d_v] per {so.b, so.h} (written; so.l unused).
 *   workspace : device buffer of at least sdpa_decode_workspace_bytes(B, h, L)
 *          bytes, 16-byte aligned, caller-owned scratch for the per-split
 *          partial results; must not overlap any tensor.
 *   Requirements: in_dt == MHA_BF16 (MHA_ENOTSUP otherwise), d_k == d_v == 64,
 *   B >= 0, h >= 1, L >= 1, pointers 16-byte aligned, strides multiples of 8
 *   elements (output: 8 bf16 or 4 fp32), o must not overlap q, k, v.
 *   The row strides of k and v must stay below 2^21 elements (a slice of
 *   512 cached rows is addressed with 31-bit byte offsets; MHA_ENOTSUP
 *   otherwise).
 *   B == 0 is a no-op.  Computed in fp32 from the bf16 inputs (no reduced-
 *   precision weights) over slices of 512 keys (256 when B*h is small); a
 *   cache of one slice is finished in one launch, longer ones are split and
 *   merged through the workspace.
 */
size_t sdpa_decode_workspace_bytes(int B, int h, int L);

mha_status sdpa_decode(mha_dtype in_dt, mha_dtype out_dt,
                       const void* q, mha_strides sq,
                       const void* k, mha_strides sk,
                       const void* v, mha_strides sv,
                       void* o, mha_strides so,
                       int B, int h, int L, int d_k, int d_v, const int* lens,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_backward -- gradients of sdpa_forward with respect to q, k and v for
 * the gradient `dout` of its output (the backward pass the pages' training
 * loops take through the attention function of The Annotated Transformer).
 * With tau = 1/sqrt(d_k), p the attention weights and D_i = dout_i . o_i:
 *   dv_j = sum_i p_ij dout_i,   ds_ij = p_ij (dout_i . v_j - D_i),
 *   dq_i = tau sum_j ds_ij k_j, dk_j = tau sum_i ds_ij q_i   (allowed pairs)
 *   q, k, v, o, dout : the forward's inputs and output and the output's
 *          gradient, all in in_dt, [B, h, L, 64] views as for sdpa_forward.
 *   dq, dk, dv : written in out_dt, same shapes as q, k, v; no overlap with
 *          each other, the inputs or the workspace.
 *   valid_lens, vl_rank, causal : the forward's masks (as sdpa_forward_ex).
 *   workspace : device buffer of at least sdpa_backward_workspace_bytes(B,
 *          h, Lq) bytes, 16-byte aligned; it receives each query's
 *          log-sum-exp and D_i.
 * Two kernels: dq accumulated per query (with each row's log-sum-exp, found
 * in the same pass), then dk and dv per key.  MHA_BF16 inputs run on bf16
 * MFMA with fp32 accumulation (the weights and ds rounded to bf16 for their
 * products, as the forward rounds its weights); MHA_F32 inputs in fp32 FMA.
 * Requirements otherwise as for sdpa_forward; for MHA_BF16 inputs each
 * (batch, head)'s rows of q, k, v, o and dout must span less than 2 GiB, as
 * must 128 rows at each one's row stride (MHA_ENOTSUP otherwise).  B == 0
 * is a no-op; Lq == 0 with B > 0 writes dk and dv as zeros (their defining
 * sums are empty) and reads nothing else.
 */
size_t sdpa_backward_workspace_bytes(int B, int h, int Lq);

mha_status sdpa_backward(mha_dtype in_dt, mha_dtype out_dt,
                         const void* q, mha_strides sq,
                         const void* k, mha_strides sk,
                         const void* v, mha_strides sv,
                         const void* o, mha_strides so,
                         const void* dout, mha_strides sdo,
                         void* dq, mha_strides sdq,
                         void* dk, mha_strides sdk,
                         void* dv, mha_strides sdv,
                         int B, int h, int Lq, int Lk, int d_k, int d_v,
                         const int* valid_lens, int vl_rank, int causal,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_backward_lse -- sdpa_backward given the forward's log-sum-exp `lse`
 * (as sdpa_forward_lse writes it: device fp32 [B, h, Lq] contiguous, 4-byte
 * aligned, not overlapping the outputs or the workspace; NULL is MHA_EINVAL
 * unless B*Lq == 0), so the weights are recomputed as exp(s_ij - lse_i)
 * rather than found by a pass of their own.  For MHA_BF16 inputs a small
 * kernel writes D_i and lse (log2 units) to the workspace, then one launch
 * runs the query-side (dq) and key-side (dk, dv) workgroups together;
 * MHA_F32 inputs take sdpa_backward's fp32 kernels, which form their own
 * statistics, and do not read lse.  B*h*Lq must stay below 2^31
 * (MHA_ENOTSUP otherwise).  Everything else as sdpa_backward; the result
 * equals sdpa_backward's up to rounding when lse is the forward's.
 */
mha_status sdpa_backward_lse(mha_dtype in_dt, mha_dtype out_dt,
                             const void* q, mha_strides sq,
                             const void* k, mha_strides sk,
                             const void* v, mha_strides sv,
                             const void* o, mha_strides so,
                             const void* dout, mha_strides sdo,
                             void* dq, mha_strides sdq,
                             void* dk, mha_strides sdk,
                             void* dv, mha_strides sdv,
                             int B, int h, int Lq, int Lk, int d_k, int d_v,
                             const int* valid_lens, int vl_rank, int causal, const float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * sdpa_decode_noalloc -- sdpa_decode for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, results and errors as sdpa_decode, minus
 * the workspace: the per-split partials live in a 16 MiB array inside the
 * library that each GPU holds from the library's load until the process ends
 * (found on a device's first call with hipGetSymbolAddress; the call neither
 * allocates nor frees).  A step needs round_up(sdpa_decode_workspace_bytes(
 * B, h, L), 256) bytes of it; larger steps (B * h * ceil(L / 256) above about
 * 63,500) return MHA_EWORKSPACE before anything is enqueued.  Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two threads) race on it and must be serialised by the caller.
 * Nothing in the array needs to start at zero.  MHA_EHIP if the array's
 * device address cannot be found.
 */
mha_status sdpa_decode_noalloc(mha_dtype in_dt, mha_dtype out_dt,
                               const void* q, mha_strides sq,
                               const void* k, mha_strides sk,
                               const void* v, mha_strides sv,
                               void* o, mha_strides so,
                               int B, int h, int L, int d_k, int d_v, const int* lens, void* stream);

/* Bytes of device workspace mha_forward needs: for MHA_BF16 the merged head
 * output [B*Lq, d_model] and the Q hi, Q lo [B*Lq, d_model] and K hi, K lo,
 * V [B*Lk, d_model] projections, all bf16 (the projected route; the on-chip
 * route uses only the first region); for MHA_F32 the projected Q, K, V and
 * the merged head output in fp32.  Each region is 256-byte aligned.  Returns
 * 0 for inconsistent arguments. */
size_t mha_workspace_bytes(mha_dtype in_dt, int B, int Lq, int Lk, int d_model, int h);

/*
 * mha_forward -- multi-head attention forward (projections, head split,
 * attention per head, head merge, output projection).
 *
 *   x_q  : [B, Lq, d_model] queries' inputs (row-major, in_dt)
 *   x_kv : [B, Lk, d_model] keys'/values' inputs; may equal x_q (self-attention)
 *   w_q, w_k, w_v, w_o : [d_model, d_model] stored [out, in] as a torch linear
 *          layer stores them (y = x W^T + b), in_dt
 *   b_q, b_k, b_v, b_o : [d_model] in_dt, or NULL for no bias
 *   out  : [B, Lq, d_model] in out_dt (written; must not overlap any input or
 *          the workspace)
 *   d_model == h * d_k; d_k must be 64.
 *   valid_lens, causal: as for sdpa_forward (masks act on keys; the same mask
 *          serves every head).
 *   workspace : device buffer of at least mha_workspace_bytes(...) bytes,
 *          256-byte aligned, owned by the caller; its contents are scratch.
 */
mha_status mha_forward(mha_dtype in_dt, mha_dtype out_dt,
                       const void* x_q, const void* x_kv,
                       const void* w_q, const void* b_q,
                       const void* w_k, const void* b_k,
                       const void* w_v, const void* b_v,
                       const void* w_o, const void* b_o,
                       void* out,
                       int B, int Lq, int Lk, int d_model, int h, int d_k,
                       const int* valid_lens, int causal,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * The inspection entry points: the attention function of The Annotated
 * Transformer ("Attention" section) returns its weights p_attn beside the
 * output, and the multi-head layer keeps them for visualisation; the d2l
 * Transformer digest's masked softmax takes valid lengths per sequence or per
 * query (its decoder trains with query i given length i + 1).
 *
 * sdpa_forward_ex -- sdpa_forward plus:
 *   vl_rank : 1 -> valid_lens is [B] (as sdpa_forward); 2 -> valid_lens is
 *             [B, Lq] row-major, one length per query, shared by every head.
 *             Ignored when valid_lens is NULL.  Other values: MHA_EINVAL.
 *             A query whose length is <= 0 weights all Lk keys uniformly.
 *   p_attn  : NULL, or a device fp32 [B, h, Lq, Lk] buffer with element
 *             strides `sp` (batch, head, query) and unit stride over keys,
 *             4-byte aligned, not overlapping any other argument.  It receives the normalised weights
 *             softmax_j(q_i . k_j / sqrt(d_k)) with masked keys exactly 0.
 * With p_attn == NULL and lengths per sequence this is sdpa_forward.  Else
 * it runs the inspection kernel, one pass over the keys for each query's
 * log-sum-exp and one for the weights (rows of at most 512 keys keep their
 * scores in registers between the two; slower than sdpa_forward, meant for
 * debugging and visualisation): for MHA_BF16 inputs
 * bf16 MFMA products with fp32 sums, the weights in fp32 and P.V with the
 * weights as two bf16 terms (about 16 significant bits); for MHA_F32 inputs
 * fp32 FMA throughout.  With MHA_BF16 inputs each (batch, head)'s rows of k
 * and v must span less than 2 GiB (MHA_ENOTSUP otherwise).
 */
mha_status sdpa_forward_ex(mha_dtype in_dt, mha_dtype out_dt,
                           const void* q, mha_strides sq,
                           const void* k, mha_strides sk,
                           const void* v, mha_strides sv,
                           void* o, mha_strides so,
                           int B, int h, int Lq, int Lk, int d_k, int d_v,
                           const int* valid_lens, int vl_rank, int causal,
                           float* p_attn, mha_strides sp, void* stream);

/* Bytes of device workspace mha_forward_ex needs on its inspection path:
 * the merged heads in in_dt, then Q [B*Lq, d_model], K and V [B*Lk, d_model]
 * in fp32, each 256-byte aligned (always >= mha_workspace_bytes).  Returns 0
 * for inconsistent arguments. */
size_t mha_workspace_bytes_ex(mha_dtype in_dt, int B, int Lq, int Lk, int d_model, int h);

/*
 * mha_forward_ex -- mha_forward plus lengths per query (vl_rank 2, valid_lens
 * [B, Lq]) and the per-head weights p_attn [B, h, Lq, Lk] (fp32, as for
 * sdpa_forward_ex).  With p_attn == NULL and lengths per sequence this is
 * mha_forward (workspace: mha_workspace_bytes); otherwise the projections
 * run to fp32 Q, K, V in the workspace (mha_workspace_bytes_ex), the
 * inspection kernel attends and writes the weights, and the output
 * projection follows as in mha_forward.
 */
mha_status mha_forward_ex(mha_dtype in_dt, mha_dtype out_dt,
                          const void* x_q, const void* x_kv,
                          const void* w_q, const void* b_q,
                          const void* w_k, const void* b_k,
                          const void* w_v, const void* b_v,
                          const void* w_o, const void* b_o,
                          void* out,
                          int B, int Lq, int Lk, int d_model, int h, int d_k,
                          const int* valid_lens, int vl_rank, int causal,
                          float* p_attn, mha_strides sp,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * mha_sublayer_forward -- the pre-norm residual sublayer around multi-head
 * attention, out = x + MHA(norm(x), kv, kv) (The Annotated Transformer,
 * sublayer connection, which applies the norm first; no dropout at
 * inference), with kv = norm(x) for self-attention (memory == NULL) or the
 * given memory [B, Lk, d_model] for source attention.
 *   norm : a layer normalisation of each row with gain ln_gain and bias
 *          ln_bias ([d_model] in in_dt, NULL meaning 1 and 0) in one of the
 *          two forms the pages print:
 *            ln_kind 0 (The Annotated Transformer's LayerNorm class):
 *              gain * (x - mean) / (std + eps) + bias, std with Bessel's
 *              correction (n - 1); the class's default eps is 1e-6;
 *            ln_kind 1 (the "Transformer" study notes' torch layer):
 *              gain * (x - mean) / sqrt(var + eps) + bias, biased variance;
 *              torch's default eps is 1e-5.
 *   x : [B, L, d_model] in in_dt; out : [B, L, d_model] in out_dt, not
 *          overlapping x, memory or the workspace.  Weights, biases,
 *          valid_lens, causal and the dtype rules as for mha_forward
 *          (memory == NULL requires Lk == L).
 *   workspace : at least mha_sublayer_workspace_bytes(...) bytes.
 * A row-wise kernel writes norm(x) to the workspace (in in_dt), the
 * attention layer runs on it, and the residual add is fused into the output
 * projection's epilogue.
 */
size_t mha_sublayer_workspace_bytes(mha_dtype in_dt, int B, int L, int Lk, int d_model, int h);

mha_status mha_sublayer_forward(mha_dtype in_dt, mha_dtype out_dt,
                                const void* x, const void* memory,
                                const void* ln_gain, const void* ln_bias, int ln_kind, float ln_eps,
                                const void* w_q, const void* b_q,
                                const void* w_k, const void* b_k,
                                const void* w_v, const void* b_v,
                                const void* w_o, const void* b_o,
                                void* out,
                                int B, int L, int Lk, int d_model, int h, int d_k,
                                const int* valid_lens, int causal,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * mha_backward -- the gradients of mha_forward's output for an output
 * gradient `dout`: the training pass the pages take through the multi-head
 * layer (The Annotated Transformer and the d2l Transformer digest train
 * these models end to end; the layer is the "Transformer" study notes'
 * multi-head attention class, four linear layers stored [out, in]).  By the
 * chain rule through each step of the forward in reverse:
 *   out = Ocat W_o^T + b_o    : dOcat = dout W_o, dW_o = dout^T Ocat,
 *                               db_o = sum over rows of dout
 *   attention per head        : dQ, dK, dV as sdpa_backward computes them
 *   Q = x_q W_q^T + b_q, ...  : dx_q = dQ W_q, dW_q = dQ^T x_q, db_q = sum dQ,
 *                               dx_kv = dK W_k + dV W_v, dW_k = dK^T x_kv, ...
 *   in_dt : MHA_BF16 only (MHA_F32 is MHA_ENOTSUP).  The gradients are fp32.
 *   x_q, x_kv, w_q, w_k, w_v, w_o, b_q, b_k, b_v, sizes, valid_lens ([B]),
 *          causal : the forward's arguments, as for mha_forward (b_o does
 *          not enter any gradient and is not taken).
 *   dout : [B, Lq, d_model] bf16, the gradient of the forward's output.
 *   dx_q : [B, Lq, d_model] fp32, the gradient through the query projection.
 *   dx_kv : [B, Lk, d_model] fp32, the gradient through the key and value
 *          projections; or NULL when x_kv == x_q (self-attention, Lq == Lk),
 *          and then dx_q receives the whole gradient of that input (the sum
 *          of both paths).
 *   dw_q, dw_k, dw_v, dw_o : [d_model, d_model] fp32, [out, in] like the
 *          weights.
 *   db_q, db_k, db_v, db_o : [d_model] fp32, all four or none (NULL).
 *   workspace : at least mha_backward_workspace_bytes(...) bytes, 256-byte
 *          aligned; its contents are scratch.
 * Outputs are 16-byte aligned (bias gradients 4-byte) and overlap no input,
 * each other or the workspace.  B * L * d_model must stay below 2^31 / 6 for
 * L = Lq and L = Lk (the stacked [dQ | dK | dV] operand's bytes index in 31
 * bits; MHA_ENOTSUP otherwise).
 * The forward is recomputed, not taken from the caller: one GEMM launch
 * projects Q, K, V (bf16), the attention forward writes the merged heads
 * (bf16) and each query's log-sum-exp, a GEMM forms dOcat (bf16), the
 * attention backward recomputes the weights from the log-sum-exp and writes
 * dQ, dK, dV (bf16) side by side, one GEMM forms the input gradients (for
 * self-attention with dx_kv == NULL a single product of [dQ | dK | dV] with
 * the stacked transposed weights), and one launch pair forms the weight
 * and bias gradients as split sums over the rows, added in a fixed order.
 * With B == 0 or Lq == 0 every weight and bias gradient and dx_kv are
 * written as zeros (empty sums).
 */
size_t mha_backward_workspace_bytes(mha_dtype in_dt, int B, int Lq, int Lk, int d_model, int h);

mha_status mha_backward(mha_dtype in_dt,
                        const void* x_q, const void* x_kv,
                        const void* w_q, const void* b_q,
                        const void* w_k, const void* b_k,
                        const void* w_v, const void* b_v,
                        const void* w_o,
                        const void* dout,
                        float* dx_q, float* dx_kv,
                        float* dw_q, float* db_q,
                        float* dw_k, float* db_k,
                        float* dw_v, float* db_v,
                        float* dw_o, float* db_o,
                        int B, int Lq, int Lk, int d_model, int h, int d_k,
                        const int* valid_lens, int causal,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The training pair: a forward that keeps what the backward needs, and a
 * backward that takes it instead of recomputing it (the saved-statistic
 * form of the backward; the pages train these models end to end).
 *
 * mha_forward_train -- mha_forward for bf16 inputs that also fills `saved`
 * (device buffer of at least mha_saved_bytes(...) bytes, 16-byte aligned,
 * caller-owned, not overlapping any input or `out`) with Q, K, V (bf16
 * [B*L, d_model] each, unscaled, biases added), the merged heads (bf16
 * [B*Lq, d_model]) and each query's log-sum-exp (fp32 [B, h, Lq]).  One GEMM
 * launch projects Q, K, V, the split-head attention kernel writes the merged
 * heads and the statistic, and the output projection follows.  Its scores
 * are single bf16 products of the stored Q and K (mha_forward keeps Q and K
 * as hi + lo pairs for large logits); the output is the oracle's
 * bf16-storage reading, and the backward's weights are recomputed from the
 * same Q, K and statistic.  Arguments, sizes and errors otherwise as
 * mha_forward (B * L * d_model below 2^31 / 6 as for mha_backward).
 *
 * mha_backward_saved -- mha_backward given `saved` from mha_forward_train
 * with the same inputs, weights, biases, lengths and causal flag (the biases
 * are then not needed: they are inside the saved Q, K, V).  Skips the
 * forward's recomputation (one GEMM and one attention launch); the
 * workspace is at least mha_backward_saved_workspace_bytes(...) bytes and
 * must not overlap `saved`.  The gradients equal mha_backward's bit for bit.
 */
size_t mha_saved_bytes(mha_dtype in_dt, int B, int Lq, int Lk, int d_model, int h);

mha_status mha_forward_train(mha_dtype in_dt, mha_dtype out_dt,
                             const void* x_q, const void* x_kv,
                             const void* w_q, const void* b_q,
                             const void* w_k, const void* b_k,
                             const void* w_v, const void* b_v,
                             const void* w_o, const void* b_o,
                             void* out,
                             int B, int Lq, int Lk, int d_model, int h, int d_k,
                             const int* valid_lens, int causal,
                             void* saved, size_t saved_bytes, void* stream);

size_t mha_backward_saved_workspace_bytes(mha_dtype in_dt, int B, int Lq, int Lk, int d_model, int h);

mha_status mha_backward_saved(mha_dtype in_dt,
                              const void* x_q, const void* x_kv,
                              const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                              const void* saved, size_t saved_bytes,
                              const void* dout,
                              float* dx_q, float* dx_kv,
                              float* dw_q, float* db_q,
                              float* dw_k, float* db_k,
                              float* dw_v, float* db_v,
                              float* dw_o, float* db_o,
                              int B, int Lq, int Lk, int d_model, int h, int d_k,
                              const int* valid_lens, int causal,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code (never NULL). */
const char* mha_status_string(mha_status s);

/*
 * Kernel timing (a profiling instrument; not part of the attention path).
 * It is the one piece of library state, and it exists only on a thread that
 * turns it on: mha_timing_enable(repeat) with repeat in 1..1000 creates that
 * thread's own pool of 4096 HIP event pairs (on its first call) and turns
 * timing on for calls made from that thread only.  Every kernel such a call
 * enqueues is then launched `repeat` times in a row, bracketed by one pair of
 * events recorded on the same stream (each kernel is a pure function of its
 * inputs, so results are unchanged; repeat > 1 amortises the gaps the events
 * themselves add).  repeat = 0 turns it off for the thread; other values
 * return MHA_EINVAL; MHA_EHIP if the events cannot be created.
 * mha_timing_read() waits for the thread's recorded events, adds their
 * elapsed times per kernel name into `total_ms` and the number of launches
 * into `count` (up to `max` entries, names are static strings), returns the
 * number of entries written and clears the record; -1 on a HIP error.
 * Event pairs beyond the pool are not recorded.  With timing off (the
 * default) the entry points keep no state and may be called from any number
 * of threads at once.  The pool lives until the process ends.
 */
mha_status mha_timing_enable(int repeat);
int mha_timing_read(const char** names, double* total_ms, int* count, int max);

#ifdef __cplusplus
}
#endif

#endif /* MHA_H */
