/*
 * fa355.h -- C ABI of libfa355: exact, IO-aware fused softmax attention for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation.  For every batch b, head h and query row i:
 *
 *     O[i]   = sum_j softmax_j(scale * q[i] . k[j]) * v[j]
 *     LSE[i] = ln sum_j exp(scale * q[i] . k[j])
 *
 * with j ranging over the keys visible to row i.  This is standard attention
 * S = Q K^T, P = softmax(S), O = P V ("FlashAttention", section "The problem:
 * the n x n score matrix"; the 1/sqrt(d) of "Flash Attention -- Module 12.3",
 * section "Definition", is the caller's `scale`).  The library computes it the
 * IO-aware way: Q, K and V are streamed tile by tile through on-chip memory and
 * the softmax is taken online, keeping a running row maximum m and running
 * denominator l and rescaling the partial output whenever m grows
 * ("FlashAttention", sections "The fix: tile through SRAM, fuse the passes" and
 * "Online softmax: the enabling trick"), so the Nq x Nkv score matrix never
 * reaches device memory.  The result equals the definition up to floating-point
 * rounding ("Flash Attention -- Module 12.3", section "Common Misconception").
 *
 * LSE is not named on the pages: it is the (m, l) pair the online softmax keeps
 * per row, folded into one natural-log value m + ln l.  It is what partial
 * results over disjoint key sets need to be merged exactly ("FlashAttention
 * 1-2-3: The IO-Aware Revolution in LLM Inference", section "The Math Behind
 * the Online Softmax Trick").
 *
 * Causal masking.  Key j is visible to query row i iff j <= i + (Nkv - Nq):
 * the lower triangle including the diagonal when Nq == Nkv, aligned to the
 * last key when Nq < Nkv (a reading; the pages show only square masks).
 * Blocks of keys that no row of a query tile can see are skipped entirely
 * ("FlashAttention 1-2-3 ...", section "FlashAttention-2: Reducing Non-Matmul
 * Overhead and Causal Efficiency").
 *
 * Data layout (all arrays row-major and contiguous, head dimension fastest):
 *     q    [B][H][Nq][d]    k, v [B][H][Nkv][d]    element type `dtype`
 *     o    [B][H][Nq][d]    element type `dtype`, or float32 with FA_OUT_F32
 *     lse  [B][H][Nq]       float32 (may be NULL: not written)
 * fa_decode is the Nq == 1 case: q and o are [B][H][d], lse is [B][H].
 *
 * Ownership.  Every pointer is device memory owned by the caller (for example
 * the storage of framework tensors).  The library allocates no device memory:
 * fa_fwd, fa_fwd_fp8 and fa_quantize_e4m3 need none; fa_decode,
 * fa_decode_paged and fa_bwd use only the caller's workspace; fa_decode_noalloc
 * uses a fixed device-resident scratch array of the library instead.  No
 * pointer is retained after a call returns.
 *
 * Execution.  Calls enqueue work on `stream` (NULL = the default stream) and
 * return without waiting; results are ready when the stream is synchronised.
 * Calls are reentrant and thread-safe.  Results are deterministic: the same
 * inputs, shapes and split count give bitwise-identical outputs (no atomics).
 *
 * Errors.  Every argument is validated on the host before any HIP call; a
 * violation returns a status code and leaves the outputs untouched.  No
 * exception or abort crosses the ABI, and there is no silent fallback to a
 * slower path: an unsupported configuration returns FA_ERR_UNSUPPORTED.  A
 * failed kernel launch returns FA_ERR_HIP.  fa_last_error() gives the
 * calling thread's message for its last non-OK return.  Faults inside a
 * kernel surface, as usual in HIP, at the next synchronisation.
 *
 * Preconditions shared by the entry points:
 *   - q, k, v, o non-NULL and 16-byte aligned; lse, when given, 4-byte aligned;
 *   - o and lse do not overlap q, k, v or each other;
 *   - d is 64 or 128 (other head dimensions: FA_ERR_UNSUPPORTED);
 *   - dtype is FA_F16 or FA_BF16, optionally OR-ed with FA_OUT_F32;
 *   - scale is finite; inputs are finite (Inf/NaN inputs: undefined results);
 *   - B, H, Nq >= 0 (a zero makes the call a no-op returning FA_OK);
 *     Nkv >= 1 whenever there is work (attention over no keys is undefined);
 *   - causal requires Nq <= Nkv, so every row sees at least one key;
 *   - B*H*N*d fits in 2^62 elements, and one head of q, k, v or o is
 *     smaller than 4 GiB (FA_ERR_UNSUPPORTED otherwise: the kernels address a
 *     head through 32-bit range-checked buffer offsets).
 */
#ifndef FA355_H
#define FA355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's opaque stream handle (identical to the typedef in hip_runtime_api.h). */
typedef struct ihipStream_t *hipStream_t;

#define FA355_VERSION 5

/* Element type of q, k, v (and of o unless FA_OUT_F32 is set). */
enum fa_dtype {
    FA_F16 = 1,  /* IEEE binary16 */
    FA_BF16 = 2  /* bfloat16 */
};

/* OR into dtype: o is written as float32 instead of the input element type. */
#define FA_OUT_F32 0x100

enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID = 1,     /* a precondition above is violated */
    FA_ERR_UNSUPPORTED = 2, /* valid request this build does not implement (e.g. d = 96) */
    FA_ERR_WORKSPACE = 3,   /* fa_decode / fa_bwd workspace missing, misaligned or too small */
    FA_ERR_HIP = 4          /* the HIP runtime reported an error (see fa_last_error) */
};

/*
 * Prefill / general forward: O and LSE for B*H heads of Nq queries against
 * Nkv keys.  `causal` non-zero applies the mask described above.  `scale`
 * multiplies every dot product before the softmax (1/sqrt(d) for the
 * textbook form).  See the file comment for layout, ownership and errors.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int Nq, int Nkv, int d, int causal, float scale, int dtype,
           hipStream_t stream);

/*
 * Forward with Q and K in FP8 for the first product: FlashAttention-3's FP8
 * mode ("FlashAttention 1-2-3 ...", section "FlashAttention-3: FP8, Async Warp
 * Overlap, and Hopper-Specific Optimizations": Q and K quantised to FP8, V and
 * O kept in 16 bits, fp32 accumulation).  The format is OCP E4M3 ("e4m3fn":
 * bias 7, largest finite value 448, no infinity).  With no scaling factor on
 * the pages, a value is quantised on its own: nearest E4M3 value, ties to
 * even, magnitudes beyond 448 (infinities included) saturated to +-448.
 *
 *   O = softmax(scale * e4m3(q) k8^T [causal]) v,   LSE as for fa_fwd
 *
 * q, v, o, lse: as for fa_fwd (dtype names the type of q and v, and of o unless
 * FA_OUT_F32).  k8: E4M3 bytes [B][H][Nkv][d] -- a cache already held in FP8,
 * or the output of fa_quantize_e4m3 on a 16-bit K.  q is quantised inside the
 * kernel as it is loaded.  Alignment, overlap and error rules as for fa_fwd.
 */
int fa_fwd_fp8(const void *q, const void *k8, const void *v, void *o, float *lse,
               int B, int H, int Nq, int Nkv, int d, int causal, float scale, int dtype,
               hipStream_t stream);

/*
 * Quantise n values of type dtype (FA_F16 or FA_BF16, no flags) at x to E4M3
 * bytes at y, with the rounding fa_fwd_fp8 applies to q.  x and y are device
 * memory, 16-byte aligned, not overlapping.  n = 0 is a no-op.
 */
int fa_quantize_e4m3(const void *x, void *y, size_t n, int dtype, hipStream_t stream);

/*
 * Decode: one query per (b, h) against Nkv cached keys and values, all visible
 * ("Flash Attention -- Module 12.3", section "Prefill vs Decode": T_q = 1
 * against a long cache).  The key range is cut into `num_splits` chunks that
 * are processed in parallel, each producing a partial softmax result, and the
 * partials are then merged exactly by their LSE values -- the split-KV scheme
 * of "FlashAttention 1-2-3 ...", section "Beyond FlashAttention: Future
 * Directions and Alternatives" (parallelising over the KV length, then a
 * reduction).  num_splits = 0 lets the library choose (fa_decode_num_splits);
 * any positive value is clamped to [1, Nkv].  The result is within rounding of
 * the definition for every split count.
 *
 * workspace: caller-owned device memory of at least
 * fa_decode_workspace_size(B, H, Nkv, d, num_splits) bytes, 16-byte aligned,
 * not overlapping any other argument.  Its contents on entry are ignored and
 * on return are unspecified.  Calls that share a workspace must be ordered on
 * one stream.  A missing, misaligned or short workspace returns
 * FA_ERR_WORKSPACE.
 */
int fa_decode(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int Nkv, int d, float scale, int dtype, int num_splits,
              void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_decode for callers that cannot allocate device memory -- code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc: the
 * same computation, kernels and split rule as fa_decode (bit-identical
 * results for the same arguments), with the split partials kept in a
 * device-resident scratch array of the library instead of a caller
 * workspace.  The caller still passes q, k, v, o and lse as for fa_decode.
 *
 * The scratch is 4 MiB (FA_DECODE_NOALLOC_SCRATCH_BYTES) per device, held
 * from the library's first use on that device until the process ends; a call
 * whose partials, B * H * splits * (d + 1) * 4 bytes (none with one split),
 * would not fit returns FA_ERR_WORKSPACE before touching the device (at the
 * automatic split count every call with B * H <= 2048 fits).  The scratch's
 * address is looked up once per device, on that device's first call (which
 * therefore should not itself be under graph capture).  The call allocates
 * nothing and frees nothing.
 *
 * Every call on one device shares that device's scratch: calls that may
 * overlap in time on one device (different streams, different host threads
 * without ordering) race on it and give undefined results; calls ordered on
 * one stream are safe.  The contents left by an earlier call are never read.
 */
#define FA_DECODE_NOALLOC_SCRATCH_BYTES (4u << 20)
int fa_decode_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                      int B, int H, int Nkv, int d, float scale, int dtype, int num_splits,
                      hipStream_t stream);

/* Bytes of workspace fa_decode needs for these arguments (0 if they are invalid,
 * or if the split kernel's grid, B * H * splits workgroups of 256 threads,
 * would exceed HIP's 2^32 - 1 work-items, which fa_decode rejects). */
size_t fa_decode_workspace_size(int B, int H, int Nkv, int d, int num_splits);

/* The split count fa_decode uses for num_splits = 0 (0 if the arguments are invalid). */
int fa_decode_num_splits(int B, int H, int Nkv, int d);

/* Page layouts of the paged cache (fa_decode_paged's `layout`). */
enum {
    FA_PAGED_HND = 0, /* k_pages, v_pages: [num_pages][H][page_size][d]: a head's slots contiguous */
    FA_PAGED_NHD = 1  /* k_pages, v_pages: [num_pages][page_size][H][d]: a slot's heads contiguous */
};

/*
 * Decode over a paged KV cache: fa_decode for B sequences whose keys and
 * values live in fixed-size pages of a shared pool, located through a block
 * table, each page being one tile of the attention ("FlashAttention 1-2-3
 * ...", sections "Integration in Major Inference Engines" and "Beyond
 * FlashAttention: Future Directions and Alternatives").  Key j < seq_lens[b]
 * of sequence b is slot j % page_size of page block_table[b][j / page_size];
 * O and LSE are the attention of q[b][h] over those seq_lens[b] keys, exactly
 * as fa_decode computes it over a contiguous cache.
 *
 *   q, o          [B][H][d] (o in q's type, or fp32 with FA_OUT_F32); lse [B][H] or NULL
 *   k_pages,
 *   v_pages       num_pages pages in `layout` (FA_PAGED_HND or FA_PAGED_NHD), q's type
 *   block_table   [B][max_pages] int32 page indices, device memory
 *   seq_lens      [B] int32 key counts, device memory
 *   max_seq_len   a host-side bound on seq_lens, 1 <= max_seq_len <= max_pages * page_size;
 *                 it sizes the key-range splits exactly as Nkv does for fa_decode
 *
 * block_table and seq_lens are read on the device, so the library cannot
 * check them: a length outside [0, max_seq_len] is clamped into it, and a
 * page index outside [0, num_pages) is clamped into the pool, so a bad table
 * yields wrong values but no access outside the arguments.  Table entries
 * past a sequence's last page are never read.  A sequence of length 0 gets
 * O = 0 and LSE = -infinity.  page_size may be any value >= 1, and
 * max_pages * page_size must stay below 2^31.
 *
 * workspace: as for fa_decode, fa_decode_workspace_size(B, H, max_seq_len, d,
 * num_splits) bytes.  q, k_pages, v_pages, o and workspace must be 16-byte
 * aligned, block_table, seq_lens and lse 4-byte aligned; o and lse must not
 * overlap any input.  Errors: FA_ERR_INVALID for bad sizes, layout, pointers
 * or overlaps; FA_ERR_UNSUPPORTED for d not in {64, 128}; FA_ERR_WORKSPACE as
 * for fa_decode.
 */
int fa_decode_paged(const void *q, const void *k_pages, const void *v_pages, const int32_t *block_table,
                    const int32_t *seq_lens, void *o, float *lse, int B, int H, int d, int num_pages,
                    int page_size, int max_pages, int layout, int max_seq_len, float scale, int dtype,
                    int num_splits, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Backward of fa_fwd: gradients dq, dk, dv of a loss L given dout = dL/do.
 * The forward keeps only its per-row statistics (LSE) rather than the softmax
 * matrix, and the backward recomputes the probabilities tile by tile from
 * them, again without writing an Nq x Nkv matrix to device memory
 * ("FlashAttention 1-2-3 ...", section "FlashAttention-1: Tiling,
 * Recomputation, and Online Softmax"; "Flash Attention -- Module 12.3",
 * section "Training": the backward is IO-aware too).  With z = scale * q.k and
 * P = exp(z - LSE), the chain rule through the definition gives
 *
 *     dv = P^T dout,   dP = dout v^T,   D_i = sum_c dout[i][c] o[i][c],
 *     dS = P * (dP - D),   dq = scale * dS k,   dk = scale * dS^T q.
 *
 * Inputs: q, k, v, o (the forward's output, in the input element type), dout
 * (like o) and lse (float32 [B][H][Nq], the forward's), all with the layouts
 * and the causal rule above.  Outputs: dq like q, dk and dv like k, in the
 * input element type or float32 with FA_OUT_F32.  The same q, k, v, causal
 * and scale as the forward call must be passed.
 *
 * workspace: caller-owned device memory of at least
 * fa_bwd_workspace_size(B, H, Nq) bytes (two float32 values per query row),
 * 16-byte aligned, not overlapping any other argument; contents ignored on
 * entry, unspecified on return; calls sharing it must be ordered on one
 * stream.  A missing, misaligned or short workspace returns FA_ERR_WORKSPACE.
 * dq, dk, dv must not overlap any input or each other.  Deterministic (no
 * atomics): the key-block and query-block passes each recompute P.
 *
 * Nq = 0: no query reaches any key, so dk = dv = 0 is written; q, o, dout,
 * lse and dq are not accessed and may be NULL.  B = 0 or H = 0: FA_OK,
 * nothing is accessed.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, void *dq, void *dk, void *dv,
           int B, int H, int Nq, int Nkv, int d, int causal, float scale, int dtype,
           void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace fa_bwd needs: 0 for Nq = 0 (no workspace is used), and 0
 * if the arguments are invalid or B * H * Nq >= 2^56 (fa_bwd rejects every
 * such call: its tensors would exceed 2^62 elements). */
size_t fa_bwd_workspace_size(int B, int H, int Nq);

/* Static, human-readable name of a status code. */
const char *fa_status_str(int status);

/* The calling thread's message for its last non-OK return ("" if none). */
const char *fa_last_error(void);

/* FA355_VERSION of the loaded library. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA355_H */
