/*
 * fa.h - fused attention forward pass (and its backward pass) for AMD
 * Instinct MI355X (gfx950).
 *
 * Computes, for every query row i of every (batch b, query head h):
 *
 *   O[b,h,i,:] = sum_j p_ij V[b,hk,j,:] / sum_j p_ij,   p_ij = exp(s_ij - max_j s_ij)
 *   LSE[b,h,i] = log(sum_j exp(s_ij)),                  s_ij = scale * (Q[b,h,i,:] . K[b,hk,j,:])
 *
 * with hk = h / (H / HKV) (grouped-query attention) and j running over the
 * keys visible to row i:
 *   causal != 0  keeps j <= i (top-left aligned, also when Sq != Sk);
 *   window  > 0  keeps j >= i - window + 1 (self included); 0 = no window.
 * A row with no visible key gets O = 0 and LSE = -inf.
 *
 * Sources: the operation and the log-sum-exp output follow the rustytorch
 * flash_attention_forward.metal kernel (online softmax, "log-sum-exp for
 * backward" output); the GQA head map and the sliding window follow the
 * forge flash_attention.metal forward kernel (FlashParams.window, hkv =
 * h / (H / HKV)); the argument set (B, H, HKV, Sq, Sk, D, scale, causal,
 * window) and the [B, H, S, D] layout follow the FlashParams uniform and
 * header comment of the boostr flash.wgsl shader. The online-softmax
 * recurrence (running max m, running sum l, rescale by exp(m_old - m_new))
 * is the one in the forge header comment; nothing of size Sq x Sk is stored.
 *
 * Entry points: the forward pass (fa_fwd, fa_fwd_ex, fa_fwd_strided,
 * fa_fwd_block_sparse, fa_fwd_noalloc) and its backward pass (fa_bwd,
 * fa_bwd_strided, fa_bwd_block_sparse), with fa_plan_splits, fa_bwd_plan,
 * fa_schedule_table, fa_status_string and fa_release.
 *
 * The library is plain C ABI: no HIP or torch types in any signature.
 */
#ifndef FA_H
#define FA_H

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of Q, K, V and O. LSE is always float32. */
enum fa_dtype {
  FA_F32 = 0,   /* float32 in and out, float32 MFMA arithmetic            */
  FA_BF16 = 1,  /* bfloat16 in and out, float32 accumulate and softmax    */
  FA_F16 = 2    /* float16 in and out, float32 accumulate and softmax     */
                /* (mixed precision: the "Support mixed precision" TODO of
                   the metal-flash-attention README)                      */
};

/* Status codes. Every argument error is detected on the host before any
 * device work is queued; nothing is written in that case. */
enum fa_status {
  FA_OK = 0,
  FA_ERR_NULLPTR = 1,   /* a required pointer is NULL                          */
  FA_ERR_SHAPE = 2,     /* a dimension < 1, or a tensor larger than 2^62 bytes */
  FA_ERR_GQA = 3,       /* H is not a multiple of HKV                          */
  FA_ERR_HEAD_DIM = 4,  /* D not in {16, 32, 48, 64, 80, 96, 128, 256}; block
                           masks: D not in {64, 128, 256}                       */
  FA_ERR_DTYPE = 5,     /* dtype not an fa_dtype value                         */
  FA_ERR_WINDOW = 6,    /* window < 0 or causal not 0/1                        */
  FA_ERR_ALIGN = 7,     /* a buffer is not 16-byte aligned                     */
  FA_ERR_HIP = 8,       /* the HIP runtime reported an error                   */
  FA_ERR_WORKSPACE = 9, /* split-K workspace could not be allocated            */
  FA_ERR_SPLITS = 10,   /* num_splits < 0 or above FA_MAX_SPLITS               */
  FA_ERR_STRIDE = 11,   /* fa_fwd_strided: a stride breaks the stride rules    */
  FA_ERR_MASK = 12      /* fa_fwd_block_sparse: mask axes are not 1 / B, 1 / HKV / H */
};

#define FA_MAX_SPLITS 64

/*
 * fa_fwd - forward pass.
 *
 *   Q    device pointer, [B, H,   Sq, D] contiguous, element type `dtype`
 *   K    device pointer, [B, HKV, Sk, D] contiguous, element type `dtype`
 *   V    device pointer, [B, HKV, Sk, D] contiguous, element type `dtype`
 *   O    device pointer, [B, H,   Sq, D] contiguous, element type `dtype` (written)
 *   LSE  device pointer, [B, H,   Sq]    contiguous, float32, natural log (written)
 *   D      head dim: 16, 32, 48, 64, 80, 96, 128 or 256 (the head dims the
 *          forge flash_attention.metal page instantiates, and 256). Dims
 *          without a kernel of their own (bf16/fp16: 16, 32, 48, 80, 96;
 *          float32: 16, 48, 80) run on the next larger kernel with the
 *          missing dims held as zeros on chip (no padded copy in memory).
 *   scale  multiplies q.k after the dot product (callers usually pass 1/sqrt(D))
 *   causal 0 or 1; window >= 0 (0 = none)
 *   stream hipStream_t to queue the work on, NULL = the null stream
 *
 * The caller owns all five buffers; all must be 16-byte aligned and must not
 * overlap O or LSE with the inputs. Every element of O and LSE is written,
 * including rows with no visible key. The call is asynchronous with respect
 * to the host; it keeps no reference to the buffers after the queued work
 * completes. Returns an fa_status code.
 *
 * Long key ranges with few query tiles are split across workgroups along the
 * key axis and merged by log-sum-exp weights; the partial results live in a
 * library-owned, stream-ordered workspace (see fa_release).
 *
 * float32 causal or windowed problems with few query tiles (fewer than two
 * per CU) run persistent workgroups over a balanced list of key-split pieces.
 * The list depends only on the shape; the first call with a new shape builds
 * it on the host and uploads it with a synchronous copy (so that call must not
 * be made during stream capture), later calls reuse it until fa_release.
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
           int B, int H, int HKV, int Sq, int Sk, int D,
           float scale, int causal, int window, int dtype, void* stream);

/*
 * fa_fwd_ex - fa_fwd with an explicit number of key-axis splits.
 *
 *   num_splits 0 = choose automatically (what fa_fwd does), 1 = never split,
 *              n = split the key range into n contiguous chunks (n is capped
 *              to the number of key tiles). At most FA_MAX_SPLITS.
 * Same arguments, ownership and errors as fa_fwd otherwise.
 */
int fa_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* LSE,
              int B, int H, int HKV, int Sq, int Sk, int D,
              float scale, int causal, int window, int dtype,
              int num_splits, void* stream);

/*
 * fa_fwd_strided - fa_fwd_ex on tensors with arbitrary batch, head and row
 * strides, e.g. the token-major [B, S, heads, D] layout of the forge
 * flash_attention.metal kernels (row stride heads * D, head stride D), or
 * views into packed QKV / KV buffers.
 *
 *   q_strides, k_strides, v_strides, o_strides
 *          host pointers to 3 element strides each: {batch, head, row}; the
 *          head dimension D is contiguous (stride 1). NULL = the contiguous
 *          [B, heads, S, D] strides of that tensor. Read during the call only.
 *   Element (b, h, i, d) of Q lives at Q + b q_strides[0] + h q_strides[1] +
 *   i q_strides[2] + d, and likewise for K and V (with the kv head) and O.
 *   LSE stays contiguous [B, H, Sq] float32.
 *
 * Stride rules (else FA_ERR_STRIDE): every stride >= 0 and a multiple of 16
 * bytes; every row stride >= D; the K and V row strides are below 2^31 / 64
 * bytes and, for D = 64, 128 and 256, multiples of D; O's rows are pairwise disjoint (checked: its
 * axes sorted by stride, each stride reaches past the extent of the smaller
 * ones). Batch or head strides of 0 (broadcast inputs) are allowed for Q, K
 * and V. O must not overlap the inputs (not checked). When all four tensors have contiguous strides the
 * call runs exactly as fa_fwd_ex. Same arguments, ownership and other errors
 * as fa_fwd_ex.
 */
int fa_fwd_strided(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int B, int H, int HKV, int Sq, int Sk, int D,
                   const long long* q_strides, const long long* k_strides,
                   const long long* v_strides, const long long* o_strides,
                   float scale, int causal, int window, int dtype,
                   int num_splits, void* stream);

/* Size of the static per-GPU workspace of fa_fwd_noalloc (68 MiB). */
#define FA_NOALLOC_SCRATCH_BYTES (68u * 1024u * 1024u)

/*
 * fa_fwd_noalloc - fa_fwd_ex for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. It calls no hipMalloc, hipFree or memory-pool routine.
 *
 * Same arguments as fa_fwd_ex; the caller still passes all five buffers.
 * The key-split partials live in a static device array of
 * FA_NOALLOC_SCRATCH_BYTES on each GPU the library runs on, held until the
 * process ends; its address is looked up on the first call on each device.
 * Differences from fa_fwd_ex:
 *   - float32 causal / windowed problems with few query tiles run one
 *     workgroup per item instead of the persistent schedule (whose device
 *     table fa_fwd_ex allocates);
 *   - num_splits = 0 takes fa_fwd_ex's automatic count, lowered until the
 *     partials (num_splits * B * H * Sq * (D + 1) float32 values, D rounded
 *     up to its kernel's tile dim) fit the array;
 *   - an explicit num_splits whose partials do not fit returns
 *     FA_ERR_WORKSPACE before any device work.
 * All calls on one GPU share its array: calls that overlap on one GPU (on
 * different streams or threads) race; calls queued in order on one stream
 * do not. Asynchronous on `stream`. Other errors as fa_fwd_ex.
 */
int fa_fwd_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                   int B, int H, int HKV, int Sq, int Sk, int D,
                   float scale, int causal, int window, int dtype,
                   int num_splits, void* stream);

/* Block-mask granularity of fa_fwd_block_sparse: query rows x keys per byte. */
#define FA_MASK_BLOCK_Q 128
#define FA_MASK_BLOCK_K 64

/*
 * fa_fwd_block_sparse - fa_fwd_ex under a programmable block mask: the block
 * sparsity of the metal-flash-attention README ("Modifications to
 * FlashAttention": block masks held in memory, covering causal and arbitrary
 * sparsity patterns).
 *
 *   block_mask  device pointer, unsigned bytes, contiguous
 *               [mask_batch][mask_heads][ceil(Sq / FA_MASK_BLOCK_Q)][ceil(Sk / FA_MASK_BLOCK_K)]
 *   mask_batch  1 (one mask for every batch entry) or B
 *   mask_heads  1 (shared), HKV (per kv head) or H (per query head)
 *
 * Key j is visible to query row i of (b, h) when the causal and window rules
 * allow it AND the mask byte of block (i / FA_MASK_BLOCK_Q, j / FA_MASK_BLOCK_K)
 * for (b, h) is nonzero. Rows left with no visible key get O = 0 and
 * LSE = -inf. Key blocks whose byte is 0 are neither read nor computed.
 * Q, K, V, O contiguous as for fa_fwd; D = 64, 128 or 256. The mask is read by the kernels on
 * `stream` (it must stay valid until they complete) and is not modified.
 * Errors as fa_fwd_ex, plus FA_ERR_NULLPTR for a NULL mask and FA_ERR_MASK
 * for other mask axis sizes. Key ranges of more than 2048 key tiles per
 * workgroup are split along the key axis automatically (FA_ERR_SHAPE if
 * FA_MAX_SPLITS splits are not enough).
 */
int fa_fwd_block_sparse(const void* Q, const void* K, const void* V, void* O, float* LSE,
                        int B, int H, int HKV, int Sq, int Sk, int D,
                        const unsigned char* block_mask, int mask_batch, int mask_heads,
                        float scale, int causal, int window, int dtype,
                        int num_splits, void* stream);

/*
 * fa_plan_splits - the number of key-axis splits fa_fwd would use for this
 * problem on the current device (1 = no split). Returns a negative fa_status
 * on argument errors. Queries the device once (HIP call), queues no work.
 */
int fa_plan_splits(int B, int H, int HKV, int Sq, int Sk, int D,
                   int causal, int window, int dtype);

/*
 * fa_bwd_plan - how fa_bwd would run this problem (contiguous tensors, no
 * block mask) on a device with num_cus compute units: host computation only
 * (no HIP call, so it also runs without a GPU). Writes 8 ints to plan:
 *   [0] the kernels' head dim (D, or the tile D is zero-padded into),
 *   [1] 1 when 16-bit inputs run the kernels' general form in place,
 *   [2] 1 when the inputs are staged into contiguous zero-padded copies,
 *   [3] 1 when fp32 runs the per-row VALU kernels (else MFMA kernels),
 *   [4] key chunks (dQ; the per-row kernels' ranges too), [5] keys per chunk,
 *   [6] query-row chunks of the MFMA dK/dV kernels, [7] rows per chunk (a
 *       multiple of 128 when [6] > 1),
 * following the backward's small-grid rules (its dQ key chunks, dK/dV row
 * chunks and fp32 head-dim staging; the reasons are in fa_bwd_api.cpp).
 * Returns FA_OK, or the argument error fa_bwd would return (FA_ERR_NULLPTR
 * for a NULL plan, FA_ERR_SHAPE for num_cus < 1).
 */
int fa_bwd_plan(int B, int H, int HKV, int Sq, int Sk, int D, int causal, int window,
                int dtype, int num_cus, int* plan);

/*
 * fa_schedule_table - the item lists of a persistent launch with nslot
 * workgroups for this problem (host computation only; no HIP call, so it
 * also runs without a GPU). Writes min(length, capacity) ints to `table`:
 * nslot + 1 offsets, then item ids (item = q_tile * units + unit, units =
 * B * H * splits; slot s runs items table[nslot + 1 + k] for k in
 * [table[s], table[s + 1])). Stores the key-split count in *num_splits when
 * that pointer is not NULL. Returns the full length, or a negative fa_status
 * on argument errors (nslot < 1, or capacity > 0 with a NULL table, gives
 * -FA_ERR_SHAPE).
 */
int fa_schedule_table(int B, int H, int HKV, int Sq, int Sk, int D,
                      int causal, int window, int dtype, int nslot,
                      int* table, int capacity, int* num_splits);

/*
 * fa_bwd - backward pass: the gradients of sum(O * dO) with respect to Q, K
 * and V, for O and LSE from fa_fwd with the same arguments. It follows the
 * backward kernels of the forge flash_attention.metal page: probabilities
 * recomputed from the saved LSE, D_i = dO_i . O_i, dS = P (dO V^T - D),
 * dQ = scale dS K, dK = scale dS^T Q and dV = P^T dO, with dK and dV summed
 * over the query heads of each kv head; per-row accumulation, no atomics
 * (deterministic).
 *
 *   Q, K, V, O, dO  device pointers, contiguous, element type `dtype`
 *                   (Q, O, dO [B, H, Sq, D]; K, V [B, HKV, Sk, D])
 *   LSE             device pointer, [B, H, Sq] float32 (the forward's output)
 *   dQ              device pointer, [B, H, Sq, D]   float32 (written)
 *   dK, dV          device pointers, [B, HKV, Sk, D] float32 (written; keys no
 *                   query sees get 0)
 *   D, scale, causal, window, dtype: as for fa_fwd; rows with LSE = -inf (no
 *   visible key) get dQ = 0 and contribute nothing.
 *
 * Contiguous tensors only (block masks: fa_bwd_block_sparse). All buffers
 * 16-byte aligned. A
 * [B, H, Sq] float32 workspace comes from the library's stream-ordered memory
 * pool (the one fa_release trims). For bf16/fp16 inputs at D = 16, 32, 48,
 * 80 or 96 the work runs on copies of Q, K, V, O, dO (and of the fp32
 * gradients) zero-padded to D = 64 or 128, also from that pool. float32
 * inputs (and D = 256) on small grids take up to 512 MiB more there for
 * partial sums, added up in a fixed order (results stay deterministic).
 * Asynchronous on `stream`. Errors as fa_fwd.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* LSE, float* dQ, float* dK, float* dV,
           int B, int H, int HKV, int Sq, int Sk, int D,
           float scale, int causal, int window, int dtype, void* stream);

/*
 * fa_bwd_strided - fa_bwd on views with arbitrary batch, head and row
 * strides, e.g. the token-major [B, S, heads, D] layout the forge
 * flash_attention.metal backward kernels address (row stride heads * D,
 * head stride D), or slices of packed QKV buffers.
 *
 *   q_strides, k_strides, v_strides, o_strides, do_strides
 *          host pointers to 3 element strides {batch, head, row} of Q, K, V,
 *          O and dO (input type), as for fa_fwd_strided; NULL = contiguous
 *   dq_strides, dk_strides, dv_strides
 *          the same for the float32 gradients dQ, dK, dV; NULL = contiguous
 *   LSE stays contiguous [B, H, Sq] float32. Strides are read during the call.
 *
 * Stride rules (else FA_ERR_STRIDE): every stride >= 0 and a multiple of 16
 * bytes, every row stride >= D, and the rows of dQ, dK and dV pairwise
 * disjoint; batch or head strides of 0 (broadcast inputs) are allowed for the
 * inputs. When every view is contiguous the call runs exactly as fa_bwd.
 * Otherwise bfloat16 and float16 views are read and written in place by the
 * kernels, as long as every row stride of Q, K, V, O, dO is at most 2^22
 * elements; fp32 views (and 16-bit ones with longer rows) are first copied to
 * contiguous rows and their gradients copied back into the views at the end
 * (stream-ordered workspace from the library's pool). Same arguments,
 * ownership and other errors as fa_bwd.
 */
int fa_bwd_strided(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, float* dQ, float* dK, float* dV,
                   int B, int H, int HKV, int Sq, int Sk, int D,
                   const long long* q_strides, const long long* k_strides,
                   const long long* v_strides, const long long* o_strides,
                   const long long* do_strides, const long long* dq_strides,
                   const long long* dk_strides, const long long* dv_strides,
                   float scale, int causal, int window, int dtype, void* stream);

/*
 * fa_bwd_block_sparse - fa_bwd for O and LSE from fa_fwd_block_sparse with the
 * same arguments: the gradients of sum(O * dO) under the block mask (the
 * programmable block masks of the metal-flash-attention README,
 * "Modifications to FlashAttention", through the backward kernels of the
 * forge flash_attention.metal page).
 *
 *   block_mask, mask_batch, mask_heads: as for fa_fwd_block_sparse (device
 *               bytes [mask_batch][mask_heads][ceil(Sq / FA_MASK_BLOCK_Q)]
 *               [ceil(Sk / FA_MASK_BLOCK_K)], contiguous; batch axis 1 or B,
 *               head axis 1, HKV or H)
 *
 * A pair (i, j) contributes only where the causal and window rules allow it
 * AND the mask byte of its block is nonzero; query and key blocks whose byte
 * is 0 are neither read nor computed, and keys no row sees get dK = dV = 0.
 * Contiguous tensors, D = 64, 128 or 256, H / HKV < 1024; other arguments,
 * workspace and errors as fa_bwd, plus FA_ERR_NULLPTR for a NULL mask and
 * FA_ERR_MASK for other mask axis sizes. The mask is read by the kernels on
 * `stream` (it must stay valid until they complete) and is not modified.
 */
int fa_bwd_block_sparse(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* LSE, float* dQ, float* dK, float* dV,
                        int B, int H, int HKV, int Sq, int Sk, int D,
                        const unsigned char* block_mask, int mask_batch, int mask_heads,
                        float scale, int causal, int window, int dtype, void* stream);

/* fa_status_string - static, human-readable text for a status code. */
const char* fa_status_string(int status);

/*
 * fa_release - return the split-K workspace pool of every device this
 * library has used to the HIP runtime and free the cached persistent-launch
 * schedules (after a device synchronisation on each device that holds some).
 * Must not be called while other threads call fa_fwd. Later calls allocate
 * again as needed.
 */
void fa_release(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
