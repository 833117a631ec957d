/*
 * fa.h -- C ABI of the exact tiled attention library (libfa.so), gfx950.
 *
 * Exact softmax attention computed tile by tile on one GPU:
 *   forward : O = softmax(scale * Q K^T [+ causal mask]) V, computed with an
 *             online softmax that keeps, per query row, the running maximum m
 *             and running sum l; only O and the fp32 log-sum-exp ledger
 *             LSE_i = scale * m_i + ln l_i are written, never the N x N matrix
 *             (page "flash-attention-backpropagation" (aiqz.cc), section
 *             前向台账; page "flash-attention-v2-sram-tiling" (aiqz.cc),
 *             section 5, the running-max / running-sum update).
 *   backward: P^ = exp(scale * Q K^T - LSE) is recomputed block by block from
 *             Q, K and the ledger; then dV = P^T dO, dP = dO V^T,
 *             D_i = rowsum(dO o O), dS = P^ o (dP - D), dQ = scale * dS K,
 *             dK = scale * dS^T Q (page "flash-attention-backpropagation",
 *             sections 反向总览, Softmax梯度 and QKV梯度).
 *
 * Layout: q, k, v, o, dO, dq, dk, dv are contiguous, d fastest, in the element
 * type named by `dtype` (FA_BF16: bfloat16, FA_FP32: float), all in the
 * layout named by `layout`: FA_LAYOUT_BHND = [B, H, N, d] (each head's rows
 * contiguous) or FA_LAYOUT_BNHD = [B, N, H, d] (each token's H heads
 * contiguous, as a projection writes them and as the PyTorch module of the
 * blog.xiaohack.org "flops" page, item 知识点13, takes its input; no transpose
 * is needed).  Any other layout value is FA_ERR_INVALID.  fa_fwd_strided and
 * fa_bwd_strided take any strides per tensor instead (views into a packed
 * projection buffer, for one).
 * lse is always float [B, H, N], natural log, in units of the scaled score
 * scale * q_i . k_j.  The causal mask keeps key j for query i iff j <= i
 * (queries and keys share the index range 0..N-1).
 *
 * Supported: d in {64, 96, 128, 256} in every call, with the dtypes each
 * call lists (fa_fwd, fa_bwd and its stages and the strided calls: FA_BF16
 * and FA_FP32); other d are FA_ERR_UNSUPPORTED; N >= 1 (any
 * N, tails are masked); B, H >= 1 with B*H*N*d < 2^31; scale any finite value
 * (negative and 0 included: S = scale * Q K^T as written; below 2^-100 in
 * magnitude every score of a row is equal to fp32 rounding); causal in {0, 1}.
 *
 * Ownership: every pointer is a device pointer owned by the caller.  The
 * library allocates and frees nothing and never synchronises; each call only
 * enqueues kernels on `stream` (a hipStream_t; 0 = the null stream) and
 * returns.  Results are valid once the stream has completed.  Outputs must not
 * alias inputs.  There is no global mutable state: concurrent calls on
 * different streams are safe if their buffers are disjoint.
 *
 * Errors: every entry point returns an fa_status.  All argument checks run
 * before any HIP call, so a rejected call has launched nothing.  A launch
 * failure reported by the HIP runtime returns FA_ERR_HIP.  fa_strerror maps a
 * status to a static string.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID = -1,      /* null or misaligned pointer, non-positive size, bad flag, bad scale */
  FA_ERR_UNSUPPORTED = -2,  /* head dim or dtype the library has no kernel for */
  FA_ERR_WORKSPACE = -3,    /* workspace missing or too small */
  FA_ERR_HIP = -4,          /* the HIP runtime reported a launch error */
  FA_ERR_SCRATCH = -5       /* fa_fwd_splitkv_noalloc: the call needs more than its static scratch */
} fa_status;

typedef enum { FA_BF16 = 0, FA_FP32 = 1 } fa_dtype;

typedef enum { FA_LAYOUT_BHND = 0, FA_LAYOUT_BNHD = 1 } fa_layout;

/*
 * How the bf16 backward forms dQ = scale * dS K (page
 * "flash-attention-backpropagation", section QKV梯度):
 *   FA_DQ_HANDOFF   the key/value-outer kernel stores the bf16 dS of each pair
 *                   of blocks, the operand its single recompute of P^ produced
 *                   (page "gsyq.cn news/1372000", 踩坑二: one recompute per
 *                   pair of blocks feeds all three gradients), into the
 *                   workspace; a query-outer kernel streams it and forms
 *                   dS K.  Fastest; needs a workspace of 2 bytes per
 *                   (query, key) pair the mask keeps (rounded up to 64 x 32
 *                   tiles): about B*H*N^2 bytes causal, 2*B*H*N^2 otherwise.
 *   FA_DQ_RECOMPUTE a query-outer kernel recomputes S, P^, dP and dS per pair
 *                   of blocks and forms dS K in registers; needs only the
 *                   per-row statistics.
 *   FA_DQ_ATOMIC    the key/value-outer kernel adds dS K into an fp32
 *                   accumulator in the workspace with atomics, and a last
 *                   kernel converts it (d = 64 and 128, no dropout; measured
 *                   slowest, kept for comparison).
 * fa_bwd, its stages and fa_bwd_dropout take the hand-off whenever
 * workspace_bytes >= fa_bwd_workspace_size(..., FA_DQ_HANDOFF) for their
 * B, H, N, d and causal, and the recompute otherwise.  The environment
 * variable FA_DQ_MODE=recompute forces the recompute, and FA_DQ_MODE=atomic
 * the atomic method (where it exists; the workspace must then hold its
 * accumulator).  The methods differ only in rounding (they round S, P^ and dS
 * at different points and sum in different orders); the hand-off and the
 * recompute are each bitwise reproducible, the atomic method is not.
 */
typedef enum { FA_DQ_HANDOFF = 0, FA_DQ_RECOMPUTE = 1, FA_DQ_ATOMIC = 2 } fa_dq_method;

/*
 * Forward pass.  Reads q, k, v; writes o (same layout and dtype) and
 * lse ([B,H,N], float).  One workgroup owns a block of query rows and streams
 * the key/value blocks through LDS, applying the online-softmax update of
 * page "flash-attention-v2-sram-tiling", section 5, with the normalisation by
 * l deferred to the end as in the NumPy demo of page
 * "flash-attention-backpropagation" (section Python 演示).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, int causal, float scale,
           void* stream, int dtype, int layout);

/*
 * fa_fwd and fa_bwd on strided views: each tensor is a [B, H, N, d] view
 * given by its base pointer and three element strides, so that element c of
 * row n of head h in batch b sits at base + b*stride_b + h*stride_h +
 * n*stride_n + c (the d elements of a row contiguous).  Q, K, V and dO as
 * slices of one packed projection [B, N, 3, H, d] (and dQ, dK, dV as slices
 * of its gradient) are such views, passed without a copy; the (B, N, H, d)
 * input of the PyTorch module of the blog.xiaohack.org "flops" page, item
 * 知识点13, is one without the packing.
 *
 * strides: host memory, 3 values (stride_b, stride_h, stride_n) per tensor:
 * fa_fwd_strided 12 for q, k, v, o; fa_bwd_strided 24 for q, k, v, o, dO,
 * dq, dk, dv (o being the forward's output, read here).  lse and the
 * workspace are those of fa_fwd and fa_bwd (lse contiguous [B, H, N]).  Each
 * stride must be >= 0, at most 2^40, and a multiple of 16 bytes (8 bf16 or 4
 * fp32 elements), with N * stride_n under 2^31 bytes (a head's rows are
 * addressed with 32-bit byte offsets) and every view within 2^62 bytes;
 * within an output view no two rows may overlap (a zero or short stride of a
 * dimension with more than one entry is rejected); otherwise FA_ERR_INVALID.
 * Inputs may repeat rows (a zero stride broadcasts).  Outputs must not
 * overlap one another or any input, as for the dense calls.  Everything else
 * (dtypes, d, sizes, scale, causal, workspace, dQ method, streams, errors) is
 * that of fa_fwd and fa_bwd, and the results are bitwise those of the dense
 * calls on the same values: the kernels are the same and only the addresses
 * differ.
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale,
                   const long long* strides, void* stream, int dtype);
int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, int causal, float scale,
                   const long long* strides, void* workspace, size_t workspace_bytes,
                   void* stream, int dtype);

/*
 * Bytes of device workspace fa_bwd needs for this shape with the given dQ
 * method (fa_dq_method): the fp32 row term D [B,H,N] and the ledger divided by
 * scale [B,H,N], plus the dS buffer (FA_DQ_HANDOFF; its size depends on
 * causal) or the fp32 dQ accumulator [B,H,N,d] (FA_DQ_ATOMIC).  The caller
 * allocates it (any 256-byte-aligned device buffer); its contents on entry do
 * not matter.  Returns 0 for arguments fa_bwd rejects, for a method that does
 * not exist there (FA_DQ_HANDOFF and FA_DQ_ATOMIC are bf16 only, FA_DQ_ATOMIC
 * d = 64 and 128 only) and for a size beyond 2^62 bytes.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d, int causal, int dtype, int dq_method);

/*
 * The dQ method (fa_dq_method) that fa_bwd and its stages (dropout = 0) or
 * fa_bwd_dropout (dropout = 1) take for these arguments, a workspace of
 * workspace_bytes bytes and the current FA_DQ_MODE; a negative fa_status for
 * arguments they reject (B, H, N < 1, an unsupported d or dtype, causal not
 * 0 or 1, dropout not 0 or 1).  Whether the workspace is large enough for the
 * method is the calls' own check (FA_ERR_WORKSPACE).
 */
int fa_bwd_dq_method(int B, int H, int N, int d, int causal, int dtype, size_t workspace_bytes, int dropout);

/*
 * The smallest workspace of fa_bwd: fa_bwd_workspace_size(B, H, N, d, causal,
 * dtype, FA_DQ_RECOMPUTE) (which does not depend on causal), or with
 * FA_DQ_MODE=atomic set the atomic method's.  A backward given this much takes
 * the recompute method.  Returns 0 for arguments fa_bwd rejects.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int dtype);

/*
 * Backward pass.  Reads q, k, v, o, dO and the ledger lse written by fa_fwd
 * with the same q, k, v, causal and scale (the recompute of P^ is exact only
 * for the ledger of that forward: page "flash-attention-backpropagation",
 * section 数值稳定).  Writes dq, dk, dv (same layout and dtype as q).  Uses `workspace`
 * (at least fa_bwd_workspace_bytes bytes; the dQ method follows from its size,
 * see fa_dq_method) as scratch; it is overwritten.  Kernels, in stream order:
 * D = rowsum(dO o O), the key/value-block-outer kernel (dK, dV, and the dS
 * buffer of the hand-off), the query-block-outer kernel (dQ).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const void* dO, const float* lse, void* dq, void* dk, void* dv,
           int B, int H, int N, int d, int causal, float scale,
           void* workspace, size_t workspace_bytes, void* stream, int dtype, int layout);

/*
 * The three stages fa_bwd runs, in this order on one stream, for callers that
 * schedule them themselves (for example to time or overlap them).  Calling
 * all three with the same arguments is exactly fa_bwd.
 *
 * fa_bwd_preprocess: D_i = sum_c dO_ic * O_ic (page
 *   "flash-attention-backpropagation", section Softmax梯度) and the ledger
 *   divided by scale, both negated, into the workspace (the product kernels
 *   start their S and dP accumulators from these values).  scale must be the
 *   one later passed to fa_bwd_dkdv and fa_bwd_dq.
 * fa_bwd_dkdv: the key/value-block-outer kernel (section QKV梯度): recomputes
 *   P^ and dS per pair of blocks and writes dk and dv (with the hand-off also
 *   the dS buffer; with the atomic method also the dQ accumulator).
 * fa_bwd_dq: dq from the dS buffer (hand-off), by the recomputing
 *   query-block-outer kernel, or by converting the accumulator (atomic).
 * Argument meaning, checks and errors are those of fa_bwd; the three calls
 * must get the same workspace and workspace_bytes, so that they take the same
 * dQ method.
 */
int fa_bwd_preprocess(const void* o, const void* dO, const float* lse, int B, int H, int N, int d,
                      float scale, void* workspace, size_t workspace_bytes, void* stream, int dtype,
                      int layout);
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse,
                void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
                void* workspace, size_t workspace_bytes, void* stream, int dtype, int layout);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO, const float* lse,
              void* dq, int B, int H, int N, int d, int causal, float scale,
              void* workspace, size_t workspace_bytes, void* stream, int dtype, int layout);

/*
 * Forward and backward with dropout on the attention probabilities (page
 * "blog.xiaohack.org/tag/flops", section 7, lists dropout inside the fused
 * softmax step; the pages define it no further).  Inverted dropout of the
 * normalised probabilities:
 *   P = softmax(scale * Q K^T [+ causal mask]), LSE as for fa_fwd (unchanged),
 *   O = (256 / (256 - drop_t)) * (P o Z) V,
 * with Z_ij = 1 (kept) or 0 (dropped).  A score is dropped with probability
 * drop_t / 256; drop_t is an integer in 0 .. 255 (0 keeps everything and
 * gives fa_fwd's O).
 *
 * Z is not stored: every kernel regenerates it from the counter-based
 * generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC 2011).  For head
 * bh = b * H + h, query i and key j: the 4x4 block (i / 4, j / 4) is one call
 * with counter (j / 4, i / 4, bh, offset) and key (seed mod 2^32,
 * seed / 2^32); Z_ij = 1 iff byte j % 4 (bits 8(j%4) .. 8(j%4)+7) of output
 * word i % 4 is >= drop_t.  The same (seed, offset) reproduces the same mask;
 * callers change offset (or seed) between independent uses.
 *
 * fa_bwd_dropout takes the O and LSE fa_fwd_dropout wrote with the same
 * q, k, v, causal, scale, drop_t, seed and offset, and writes dq, dk, dv of
 * the loss sum(dO o O) for that mask:
 *   D_i = sum_c dO_ic O_ic,  dP = (256 / (256 - drop_t)) * Z o (dO V^T),
 *   dS = P o (dP - D 1^T),  dV = (256 / (256 - drop_t)) (P o Z)^T dO,
 *   dQ = scale dS K,  dK = scale dS^T Q.
 *
 * bf16 only (no dtype argument); d in {64, 96, 128, 256}.  B, H, N, causal,
 * scale, layout, pointers, alignment, ownership, streams and errors are those
 * of fa_fwd and fa_bwd; the workspace is fa_bwd's, and its size chooses the
 * hand-off (the stored dS carries the mask) or the recompute (which
 * regenerates it) as there.  drop_t outside 0 .. 255 is FA_ERR_INVALID.
 * FA_DQ_MODE=atomic is ignored (there is no atomic dropout kernel).
 */
int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, int causal, float scale,
                   int drop_t, unsigned long long seed, unsigned offset, void* stream, int layout);
int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                   const void* dO, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, int causal, float scale,
                   int drop_t, unsigned long long seed, unsigned offset,
                   void* workspace, size_t workspace_bytes, void* stream, int layout);

/*
 * Forward with FP8 inputs: q, k, v hold OCP e4m3fn codes (1 byte per
 * element: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; largest finite 448) in the layout named by `layout`, standing
 * for Q = descale_q * q and so on (per-tensor descales, finite and > 0).
 * Writes o in bf16 (same layout) and lse as fa_fwd does, for
 * O = softmax(scale * Q K^T [+ causal mask]) V.
 *
 * The method is fa_fwd's (page "flash-attention-v2-sram-tiling", section 5)
 * on the FP8 matrix instructions, the FP8 forward the pages attribute to
 * FlashAttention-3 (page "data.6616ai.com flash-attention").  S comes from
 * the FP8 matrix instruction, whose dot products of codes are within
 * 2^-14 * sum_c |q_c k_c| of the exact sum (measured), so LSE is within
 * 1e-3 + 2^-14 * |scale| * max_j sum_c |q_ic k_jc| of the exact value; the
 * probabilities are rounded to e4m3 for the P V product (relative error at
 * most 2^-4 each), so O carries an error of up to about 2^-4 * max|V|.
 *
 * Supported: d in {64, 96, 128, 256}; B, H, N, causal, scale, layout,
 * ownership, streams and errors as for fa_fwd.
 * Pointers must be 16-byte aligned (lse 4-byte).
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, int causal, float scale,
               float descale_q, float descale_k, float descale_v, void* stream, int layout);

/*
 * Forward for Nq query rows against Nk key/value rows per head (the decode
 * shape: a few new tokens against a long key/value cache), with the keys of
 * each head cut into ranges that separate workgroups process at once.
 *
 * q, o: [B, H, Nq, d] (or [B, Nq, H, d]); k, v: [B, H, Nk, d] (or
 * [B, Nk, H, d]), all bf16, in the layout named by `layout`; lse: float
 * [B, H, Nq].  With causal = 1 the queries are the last Nq positions of the
 * sequence: query i keeps key j iff j <= i + Nk - Nq (requires Nq <= Nk; with
 * Nq == Nk this is fa_fwd's mask).  The results are those of the plain
 * definition, as for fa_fwd.
 *
 * Each range runs the online softmax of page "flash-attention-v2-sram-tiling"
 * (aiqz.cc), section 5, and leaves its O and its LSE in the workspace; a
 * second kernel joins the ranges per row with the rule for merging partial
 * softmax results (same page, quiz question 10: the larger maximum, each
 * partial sum rescaled to it).
 *
 * num_splits: key ranges per head; 0 lets the library choose (about 1024
 * workgroups in all, at least 128 keys per range, at most 256 ranges).
 * Ranges are whole 32-key tiles and none is left empty, so fewer ranges than
 * asked may be used.  The workspace must hold
 * fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, d, num_splits) bytes (same
 * num_splits), 256-byte aligned; its contents on entry do not matter (the
 * size function returns 0 for shapes, d or num_splits that fa_fwd_splitkv
 * rejects).  Supported: dtype FA_BF16 only (FA_ERR_UNSUPPORTED otherwise), d in
 * {64, 96, 128, 256}, 0 <= num_splits <= 1024.  Errors, ownership and streams as for
 * fa_fwd; a missing or small workspace is FA_ERR_WORKSPACE.
 */
size_t fa_fwd_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits);
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, int causal, float scale, int num_splits,
                   void* workspace, size_t workspace_bytes, void* stream, int dtype, int layout);

/*
 * fa_fwd_splitkv without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  The per-range
 * partial results live in a static device array of the library,
 * FA_SPLITKV_NOALLOC_MAX_BYTES bytes on each GPU it runs on, held until the
 * process ends; its address on a device is looked up (hipGetSymbolAddress)
 * on the first call there.  Arguments, checks and results are fa_fwd_splitkv's
 * (the same kernels run; outputs are bit-identical to fa_fwd_splitkv with the
 * same num_splits).  A call whose fa_fwd_splitkv_workspace_bytes exceeds
 * FA_SPLITKV_NOALLOC_MAX_BYTES returns FA_ERR_SCRATCH and launches nothing
 * (fewer ranges, num_splits, need less).  All calls on one GPU share the
 * array: calls that overlap in time on one GPU (different streams, or host
 * threads) race on it and must be serialised by the caller.  The array needs
 * no clearing: each call writes every partial result it reads.
 */
#define FA_SPLITKV_NOALLOC_MAX_BYTES (32u * 1024u * 1024u)
int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, int causal, float scale, int num_splits,
                           void* stream, int dtype, int layout);

/*
 * The split-key-range forward with FP8 inputs: fa_fwd_splitkv's shapes,
 * masks, ranges, workspace rules and results, with q, k, v given as e4m3fn
 * codes and per-tensor descales as in fa_fwd_fp8 (decoding against an FP8
 * key/value cache reads half the bytes of bf16).  Ranges are whole 64-key
 * tiles; the workspace must hold fa_fwd_splitkv_fp8_workspace_bytes(...)
 * bytes for the same num_splits.  Accuracy as fa_fwd_fp8.  Supported: d in
 * {64, 96, 128, 256}; other arguments and errors as for fa_fwd_splitkv and
 * fa_fwd_fp8 (fa_fwd_splitkv_fp8_workspace_bytes returns 0 for any other d).
 */
size_t fa_fwd_splitkv_fp8_workspace_bytes(int B, int H, int Nq, int Nk, int d, int num_splits);
int fa_fwd_splitkv_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Nq, int Nk, int d, int causal, float scale,
                       float descale_q, float descale_k, float descale_v, int num_splits,
                       void* workspace, size_t workspace_bytes, void* stream, int layout);

/* Static, human-readable text for a status code. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
