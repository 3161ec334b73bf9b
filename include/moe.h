/*
 * moe.h -- C ABI of a routed-expert Mixture-of-Experts layer whose experts are
 * stored as 4-bit group-64 affine records, for AMD Instinct MI355X (gfx950).
 *
 * The layer (one call of moe_forward, T tokens of width H):
 *   1. router:   l[t,e] = sum_h x[t,h] * Wr[e,h] + beta[e]       (8-bit Wr)
 *   2. select:   ids[t,:] = the top_k experts by logit, ordered by
 *                (logit descending, expert index ascending); ties go to the
 *                lowest index.
 *   3. weights:  p[t,j] = softmax over the top_k selected logits.
 *   4. experts:  FFN_e(x) = Wd_e (SiLU(Wg_e x) * (Wu_e x)),  SiLU(z) = z/(1+e^-z)
 *   5. combine:  y[t] = sum_j p[t,j] FFN_{ids[t,j]}(x[t])  [+ FFN_shared(x[t])]
 * Sources: TurboFieldfare page ("Gemma 4 26B'yi 2GB RAM ile ...") sections
 * "Belleği azaltan çalışma yapısı" (MLX affine 4-bit, group 64; 8-bit router;
 * 4-bit shared and routed experts) and "Token üretim süreci" (router on the GPU
 * from resident weights, top-8 ids, shared-expert branch computed alongside,
 * shared and routed outputs combined, prefill in chunks of at most 128 tokens);
 * WASTE page ("Kimi K3'ü 29 GB RAM'de ...") section "Disk streaming mimarisi"
 * (one expert = one 4 KiB-aligned record with gate, up and down contiguous;
 * magic, expert id and offsets are checked before a record is used) and section
 * "Önceden okuma ve router tahmini" (16 expert ids per layer; running the next
 * layer's router one residual ahead changes neither the selected experts nor
 * the output).
 *
 * ---------------------------------------------------------------------------
 * Record format (normative)
 * ---------------------------------------------------------------------------
 * Affine quantization, group 64 along each matrix's input (reduction) axis:
 *     W[r, c] = s[r, c/64] * q[r, c] + b[r, c/64]
 * q unsigned (4-bit: 0..15, 8-bit: 0..255); s and b are IEEE fp16 (subnormals
 * are values, never flushed).  All multi-byte fields are little-endian.
 *
 * Tiled matrix.  A matrix of R rows (outputs) by C columns (inputs), R and C
 * multiples of 64, is stored as (R/64) * (C/64) tiles in row-block-major order:
 * tile (rb, g) covers rows rb*64 .. rb*64+63 and columns g*64 .. g*64+63 and
 * starts at byte ((rb * (C/64)) + g) * TILE_BYTES.
 *   4-bit tile (TILE_BYTES = 2304):
 *     bytes [h*1024 + r*16 + j], h in {0,1}, r in 0..63, j in 0..15:
 *         low nibble  = q[rb*64 + r, g*64 + h*32 + 2j]
 *         high nibble = q[rb*64 + r, g*64 + h*32 + 2j + 1]
 *     bytes [2048 + 4r .. 2048 + 4r + 3]: s[rb*64 + r, g] (fp16), then
 *         b[rb*64 + r, g] (fp16)
 *   8-bit tile (TILE_BYTES = 4352):
 *     byte  [c4*1024 + r*16 + j], c4 in 0..3: q[rb*64 + r, g*64 + c4*16 + j]
 *     bytes [4096 + 4r ..]: s then b, as above.
 * (Each 16-byte piece is one row's run of consecutive columns, and 64 rows'
 * pieces are adjacent, so one wave64 load of 16 bytes per lane reads 1 KiB
 * of contiguous memory.)
 *
 * Expert record (4-bit).  hidden H, intermediate I (both multiples of 64):
 *   [0, 256)   header:
 *       u32 magic = 0x58455251 ("QREX"), u32 version = 1,
 *       i32 expert_id (index in the bank; -1 for the shared expert),
 *       u32 hidden, u32 inter, u32 group = 64, u32 bits = 4, u32 tile_rows = 64,
 *       u64 gate_off, u64 up_off, u64 down_off, u64 end_off,
 *       u32 payload_crc32 (at byte 64): CRC-32 of bytes [gate_off, end_off)
 *           with zlib's polynomial and conditioning (reflected 0xEDB88320,
 *           initial value and final xor 0xFFFFFFFF),
 *       u32 hflags (at byte 68): bit 0 set iff payload_crc32 is present (else
 *           payload_crc32 is 0); other bits zero,
 *       rest zero.
 *   gate: tiled 4-bit matrix I x H at gate_off = 256
 *   up:   tiled 4-bit matrix I x H at up_off   = gate_off + (I/64)(H/64)*2304
 *   down: tiled 4-bit matrix H x I at down_off = up_off   + (I/64)(H/64)*2304
 *   end_off = down_off + (H/64)(I/64)*2304; the record is padded with zeros to
 *   a multiple of 4096 bytes.  A bank is E records at a fixed stride
 *   (a multiple of 4096, >= end_off).
 * Router: one tiled 8-bit matrix of ceil(E/64)*64 rows by H columns; rows
 * >= E are padding and never read as experts.
 *
 * ---------------------------------------------------------------------------
 * Ownership, streams, errors
 * ---------------------------------------------------------------------------
 * Every buffer is caller-owned device memory unless stated otherwise.  The
 * library owns only the context.  Weight pointers passed to moe_set_weights
 * are borrowed until the next moe_set_weights or moe_close and are never
 * written or freed.  All device work of a call is ordered on the caller's
 * hipStream_t (passed as void*, NULL = the null stream): it starts after work
 * already enqueued there and finishes before work enqueued later.  Inside a
 * forward, the 128-row matrix-core kernels (batches with experts of 24+ rows)
 * run on a stream the context owns, forked
 * from and joined back into the caller's stream with events (so a forward can
 * be captured into a HIP graph).  moe_forward performs no host synchronisation
 * and no allocation.  A context is not thread-safe and
 * two calls on one context must not overlap on different streams (they share
 * the workspace).  Functions return MOE_OK (0) or a negative status; the
 * context keeps a message for the last failure (moe_last_error).  Asynchronous
 * kernel faults surface on a later call or synchronisation, as HIP reports them.
 */
#ifndef QREB_MOE_H
#define QREB_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK            0
#define MOE_EINVAL       (-1)   /* bad argument: null pointer, size out of range */
#define MOE_EUNSUPPORTED (-2)   /* shape or option this build does not handle    */
#define MOE_ENOMEM       (-3)   /* workspace too small                           */
#define MOE_EBADRECORD   (-4)   /* a record header failed validation             */
#define MOE_ESTATE       (-5)   /* call out of order (forward before weights)    */
#define MOE_EHIP         (-6)   /* a HIP runtime call failed                     */

#define MOE_BF16 1              /* x dtype: bf16 [T, H]                           */
#define MOE_F32  2              /* x dtype: fp32 [T, H] (e.g. a residual stream)  */
/* Input precision and range.  The router computes its logits from x at fp32
 * accuracy (bf16 x converts to fp16 exactly; fp32 x is split into fp16 hi and
 * lo halves that both enter the dot products).  The expert FFNs take x rounded
 * once to fp16 (round to nearest even; exact for bf16 x inside fp16's range),
 * dequantize the matrix-core paths' weights to fp16 (one rounding), and store
 * h = SiLU(Wg x) * (Wu x) in fp16; every sum is fp32.  Supported inputs are
 * finite with |x| <= 65504 and |h| <= 65504 (fp16's largest finite value; a
 * larger value becomes +-inf in the fp16 staging); magnitudes below 2^-14 keep
 * an absolute precision of 2^-25 (fp16 subnormals) and below 2^-25 become 0.
 * With MOE_F_RMSNORM the layer's input has RMS 1, so |x| <= sqrt(H). */

#define MOE_F_SHARED  1u        /* config flag: an always-on shared expert exists */
#define MOE_F_RMSNORM 2u        /* config flag: the layer runs on x / sqrt(mean(x^2) + 1e-6),
                                   per token (a parameter-free pre-norm, for residual stacks) */
#define MOE_F_VERIFY  4u        /* config flag: moe_set_weights checks every record's
                                   payload_crc32 on the GPU (WASTE page, "Disk streaming
                                   mimarisi": a crc32 of the payload, checked on request) */

#define MOE_ABI_VERSION 1

typedef struct moe_ctx moe_ctx;

/* Layer shape, fixed for the life of a context. */
typedef struct moe_config {
    uint32_t struct_size;   /* sizeof(moe_config) */
    int32_t  hidden;        /* H, multiple of 64, 64..16384 */
    int32_t  n_experts;     /* E, 1..1024 */
    int32_t  top_k;         /* k, 1..min(E, 32) */
    int32_t  inter;         /* I, multiple of 64, 64..16384 */
    int32_t  shared_inter;  /* Is, multiple of 64; read only with MOE_F_SHARED */
    int32_t  group;         /* must be 64 */
    int32_t  max_tokens;    /* largest T a forward may pass, 1..65536 */
    int32_t  device;        /* HIP device ordinal the context runs on */
    uint32_t flags;         /* MOE_F_SHARED | MOE_F_RMSNORM | MOE_F_VERIFY */
} moe_config;

/* Weights and workspace, all device pointers (borrowed). */
typedef struct moe_weights {
    uint32_t    struct_size;     /* sizeof(moe_weights) */
    const void *router;          /* tiled 8-bit router matrix (see format) */
    const float *router_bias;    /* fp32 [E] added to the logits, or NULL */
    const void *bank;            /* E expert records */
    uint64_t    record_stride;   /* bytes between records, multiple of 4096 */
    const void *shared_record;   /* shared-expert record, NULL iff no MOE_F_SHARED */
    void       *workspace;       /* >= moe_workspace_bytes(cfg) bytes, 256-aligned; or
                                    NULL with workspace_bytes 0: the context then runs
                                    moe_forward_noalloc only */
    uint64_t    workspace_bytes;
} moe_weights;

/* Bytes of device workspace a context with this config needs (0 if the config
 * is invalid).  Pure host computation. */
uint64_t moe_workspace_bytes(const moe_config *cfg);

/* Validate cfg and create a context on cfg->device: the "open the model" step
 * of the engine API the WASTE page lists (section "WASTE'in hedefi ve uygulama
 * biçimi": open, set the RAM cap, generate, save a session, close), for one
 * layer.  The context owns a side stream and two events (default priority).
 * *out is set only on success.  Errors: MOE_EINVAL (null or struct_size
 * mismatch), MOE_EUNSUPPORTED (shape outside the ranges above, group != 64),
 * MOE_EHIP. */
int moe_open(const moe_config *cfg, moe_ctx **out);

/* Bind weights.  Copies every record header (and the shared one) to the host
 * with one synchronous copy on `stream`, validates each with
 * moe_check_record_header (magic, expert id and offsets are checked before a
 * record is ever used: WASTE page, "Disk streaming mimarisi"), and initialises
 * the workspace's counters.  With MOE_F_VERIFY it also computes the CRC-32 of
 * every record's payload on the GPU (moe_crc32's kernel, through the static
 * scratch that moe_forward_noalloc uses, so it must not overlap such a call on
 * the same GPU) and refuses a record whose checksum is absent or differs.  On
 * any failure the context keeps no weights (a later forward gives
 * MOE_ESTATE): it refuses rather than computes from unvalidated records.
 * Errors: MOE_EINVAL, MOE_EBADRECORD, MOE_ENOMEM (workspace too small),
 * MOE_EHIP. */
int moe_set_weights(moe_ctx *ctx, const moe_weights *w, void *stream);

/* Run the layer on T = n_tokens rows of x (x_dtype MOE_BF16 or MOE_F32,
 * row-major [T, H], 16-byte aligned): the "generate" step of the engine API, one layer of it
 * (router on the GPU from resident weights, top-k, routed and shared experts,
 * combine: TurboFieldfare page, "Token üretim süreci").  Two arguments go
 * beyond the layer itself: `residual` fuses the residual add of a stack, and
 * `lookahead_next` is the WASTE page's next-layer router run one residual
 * ahead ("Önceden okuma ve router tahmini"); a flag in the config would have
 * left the next layer's context unnamed.  Writes y (fp32 [T, H]) = layer(x), or residual +
 * layer(x) when residual (fp32 [T, H]) is non-NULL -- the residual stream
 * update r_{l+1} = r_l + y_l of a stack of layers (with MOE_F_RMSNORM the layer
 * sees the normalized x, the residual add does not); y may alias residual (an
 * in-place update), and with fp32 x also x.  ids_out (int32 [T, k]) and p_out
 * (fp32 [T, k]) receive the selection when non-NULL.  If lookahead_next is a
 * context of the same hidden size and flags with weights bound, its router also
 * runs on this x ("one residual ahead") and its next forward orders expert work by
 * that prediction; the selected experts and every output are unchanged by it.
 * T = 0 is a no-op.  Errors: MOE_EINVAL (null x/y, misaligned x, T < 0 or >
 * max_tokens, bad dtype, mismatched lookahead context), MOE_ESTATE (no
 * weights), MOE_EHIP (launch failure). */
int moe_forward(moe_ctx *ctx, const void *x, int32_t x_dtype, int32_t n_tokens,
                float *y, const float *residual, int32_t *ids_out, float *p_out,
                moe_ctx *lookahead_next, void *stream);

/* Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The layer of moe_forward, computed by the same kernels (so
 * bitwise the same y, ids and p), but its workspace is the library's static
 * scratch array of MOE_NOALLOC_SCRATCH_BYTES on the context's GPU (each GPU
 * the library runs on holds one until the process ends) instead of the bound
 * workspace; the call allocates nothing.  Every call on a GPU shares that
 * GPU's array, which keeps the last call's contents: each call clears what
 * must start at zero itself, and calls that overlap on one GPU (on two
 * streams or from two threads, whatever their contexts) race.  There is no
 * lookahead argument (a prediction lives in the next layer's own workspace).
 * A context bound with workspace NULL and workspace_bytes 0 runs only this
 * call (moe_forward and moe_router_logits give MOE_ESTATE) and cannot be
 * another forward's lookahead context.  Errors: as moe_forward, and
 * MOE_ENOMEM when a forward of n_tokens tokens needs more than
 * MOE_NOALLOC_SCRATCH_BYTES (moe_workspace_bytes of the config with
 * max_tokens = n_tokens). */
#define MOE_NOALLOC_SCRATCH_BYTES (64ull << 20)
int moe_forward_noalloc(moe_ctx *ctx, const void *x, int32_t x_dtype, int32_t n_tokens,
                        float *y, const float *residual, int32_t *ids_out, float *p_out,
                        void *stream);

/* Router step only: logits fp32 [T, E] (including router_bias), of the
 * normalized rows when the context has MOE_F_RMSNORM.  Same argument rules as
 * moe_forward. */
int moe_router_logits(moe_ctx *ctx, const void *x, int32_t x_dtype, int32_t n_tokens,
                      float *logits, void *stream);

/* Tuning knob for the expert paths.  An expert's row count is the number of
 * tokens routed to it in one forward (T for the shared expert).  Rows below
 * mfma_min_rows take the streaming dot-product path; rows in
 * [mfma_min_rows, wide_min_rows) take the matrix-core path in 32-row tiles;
 * rows >= wide_min_rows take it in 128-row tiles.  Defaults: 4 and 24, or 3
 * and 24 when hidden >= 4096.
 * mfma_min_rows = 1 sends every expert to the matrix cores; values above
 * max_tokens keep them all on the streaming path.  Never changes the selected
 * experts.  Errors: MOE_EINVAL unless 1 <= mfma_min_rows <= wide_min_rows. */
int moe_set_path_rows(moe_ctx *ctx, int32_t mfma_min_rows, int32_t wide_min_rows);

/* Tuning knob for the 32-row tiles.  A tile can be split over workgroups by K
 * (each of a workgroup's four waves takes a quarter of the K groups of the
 * same 32 or 64 columns, and the partial sums are added in a fixed order) or
 * by columns (each wave takes its own columns over all K groups, so the
 * waves share the token rows and a workgroup covers four times the weights).
 * A forward takes the column split when the most 32-row tiles its batch size
 * allows would give min_workgroups workgroups or more that way (for each of
 * the gate/up and the down launch).  Default: four times the device's
 * compute-unit count.  0 always splits by columns; INT32_MAX never.
 * Both splits give the same outputs up to the order of the fp32 sums over K
 * (the selection is unchanged).  Errors: MOE_EINVAL if min_workgroups < 0. */
int moe_set_narrow_split(moe_ctx *ctx, int32_t min_workgroups);

/* Kernel timing (measurement aid).  moe_profile_start creates event pairs for
 * up to max_calls forwards; each later moe_forward on a stream that is not
 * being captured into a graph records one pair around each kernel it launches,
 * on the stream it runs on.  moe_profile_read waits for the
 * recorded events, writes the average milliseconds per launch of each kernel
 * slot into avg_ms[0 .. n_slots-1] (0 for a slot never launched) and the number
 * of profiled forwards into *n_calls, then stops profiling.  Slots:
 * 0 router+top-k+bucketing, 1 gate/up launch of the streaming path (which
 * also carries the 32-row matrix-core tiles), 2 down launch of the same,
 * 3 matrix-core gate/up (128-row tiles), 4 matrix-core down (128-row tiles),
 * 5 combine, 6 expert-cache plan and fill (demand), 7 reserved (always 0).
 * Errors: MOE_EINVAL, MOE_EHIP. */
#define MOE_PROFILE_SLOTS 8
int moe_profile_start(moe_ctx *ctx, int32_t max_calls);
/* moe_profile_start for the slots whose bit is set in slot_mask only (bit i =
 * slot i): the others record no events, so a timed region carries event pairs
 * only around the kernels it measures (moe_profile_read gives 0 for them).
 * moe_profile_start profiles every slot.  Errors: MOE_EINVAL (also for a
 * mask of 0 or with bits past MOE_PROFILE_SLOTS), MOE_EHIP. */
int moe_profile_start_slots(moe_ctx *ctx, int32_t max_calls, uint32_t slot_mask);
int moe_profile_read(moe_ctx *ctx, float *avg_ms, int32_t *n_calls, int32_t n_slots);

/* Free the context (NULL is a no-op): the "close" step of the engine API
 * (WASTE page, "WASTE'in hedefi ve uygulama biçimi").  Does not touch
 * borrowed memory. */
void moe_close(moe_ctx *ctx);

const char *moe_strerror(int code);
const char *moe_last_error(const moe_ctx *ctx);

/* Host-only validation of one record header (header_bytes >= 256 host bytes):
 * magic, version, expert_id == expected_id (-1 for the shared expert), hidden
 * and inter equal to the config's (inter = shared_inter when expected_id is -1),
 * group 64, bits 4, tile_rows 64, section offsets exactly as the format fixes
 * them with end_off <= record_stride, hflags 0 or 1 (payload_crc32 0 when 0),
 * and the reserved bytes zero.  It cannot see a wrong payload_crc32: that is
 * what MOE_F_VERIFY checks.  Returns MOE_OK or
 * MOE_EBADRECORD / MOE_EINVAL.  Touches no GPU. */
int moe_check_record_header(const void *header, uint64_t header_bytes,
                            const moe_config *cfg, int32_t expected_id,
                            uint64_t record_stride);

/* ---------------------------------------------------------------------------
 * Banks larger than HBM: an expert cache per layer
 * ---------------------------------------------------------------------------
 * The bank given to moe_set_weights may be pinned, mapped host memory (e.g.
 * hipHostMalloc); the kernels then read it over PCIe, unless the context has an
 * expert cache.  With one, a forward computes only on records in a bounded
 * set of HBM slots (TurboFieldfare page, "Token üretim süreci": the router's
 * expert ids are compared with a 16-slot LFU cache per layer, misses are read
 * in, then the experts run; WASTE page, "RAM bütçesi ve dar performans
 * aralığı": the expert cache is bounded, and a budget below one token's
 * working set is refused).  After the top-k a one-workgroup plan looks the
 * selected experts up; missing ones take the slots that sort first by
 * (free, then fewest forwards that selected their expert, then least recently
 * used, then lowest slot), never a slot whose expert this forward selects;
 * a copy kernel then reads the missing records from the bank into their
 * slots, and the expert kernels read them there.  All of it is decided on the
 * GPU, ordered on the caller's stream: no host synchronisation, no
 * allocation.  The selected experts, y, ids and p are bitwise those of the
 * same context without a cache, and each forward reads the same record bytes
 * from HBM; what the cache adds is the copies, which moe_cache_stats counts.
 *
 * With MOE_CACHE_PREFETCH, a forward of the previous layer that names this
 * context as lookahead_next prefetches this layer's predicted experts (its
 * router run one residual ahead, WASTE page, "Önceden okuma ve router
 * tahmini") into this cache on a copy stream this context owns, overlapping
 * that layer's compute; this context's next forward waits for the copies
 * before its own plan.  A prefetch never evicts for itself a slot whose expert
 * it predicts, and a record prefetched but not used is evicted first.
 * MOE_CACHE_PREFETCH_TOP(p) (with MOE_CACHE_PREFETCH, 1 <= p <= k) prefetches
 * only the p highest-ranked of each token's k predicted experts (the WASTE
 * page prefetches the top 6 of its router's 8); without it, all k.
 *
 * moe_set_cache: flags is 0 or MOE_CACHE_PREFETCH, optionally with
 * MOE_CACHE_PREFETCH_TOP(p); slots is device memory of slots_bytes >=
 * n_slots * record_stride bytes (256-aligned, caller-owned, borrowed until the next
 * moe_set_cache, moe_set_weights or moe_close), n_slots in [min(E,
 * max_tokens * k), E]; slots NULL or n_slots 0 removes the cache.  The cache
 * starts empty, its counters at zero.  It needs the bound workspace (its
 * state lives there); moe_set_weights removes it, and moe_forward_noalloc
 * refuses a context that has one.  Errors: MOE_ESTATE (no weights or no
 * workspace), MOE_ENOMEM (too few slots or bytes), MOE_EINVAL (also unknown
 * flags, or a prefetch depth without MOE_CACHE_PREFETCH or above k), MOE_EHIP.
 *
 * moe_cache_stats: the counters since moe_set_cache, into out[0 .. n-1]
 * (waits for the stream): 0 forwards, 1 experts selected, 2 demand hits,
 * 3 demand misses, 4 bytes copied on demand, 5 records prefetched, 6 bytes
 * prefetched, 7 prefetched records later selected, 8 prefetched records
 * evicted unused, 9..15 zero.  Errors: MOE_ESTATE (no cache), MOE_EINVAL,
 * MOE_EHIP. */
#define MOE_CACHE_PREFETCH 1u
#define MOE_CACHE_PREFETCH_TOP(p) ((((uint32_t)(p)) & 0xffu) << 8)
#define MOE_CACHE_STATS 16
int moe_set_cache(moe_ctx *ctx, void *slots, uint64_t slots_bytes, int32_t n_slots,
                  uint32_t flags, void *stream);
int moe_cache_stats(moe_ctx *ctx, uint64_t *out, int32_t n, void *stream);

/* ---------------------------------------------------------------------------
 * 3-bit residual-VQ matrices (WASTE page, "Quantization ve doğruluk")
 * ---------------------------------------------------------------------------
 * The WASTE engine's expert codec: every run of 8 consecutive weights of a
 * row is the sum of one 8-vector from each of three 256-entry codebooks
 * (residual vector quantization in three stages), so a weight costs 3.00 bits
 * (three 8-bit indices per 8 weights).  The product never rebuilds the
 * matrix: it builds per-input-row tables of the inner products of every
 * codebook entry with every 8-column run of x, and sums three table lookups
 * per run of each row: the three lookups and two additions per run of 8
 * weights that the page counts.
 *
 * Matrix layout: R rows by K columns (multiples of 64), (R/64) * (K/64) tiles
 * of MOE_RVQ_TILE_BYTES in row-block-major order; byte s*512 + r*8 + j of tile
 * (rb, g) is the stage-s index (0..255) of row rb*64 + r's run j, i.e. of its
 * columns g*64 + 8j .. g*64 + 8j + 7.  Codebooks: fp16 [3][256][8] (stage,
 * entry, dimension), 16-byte aligned:
 *     W[r, 8j' + d] = C[0][i0][d] + C[1][i1][d] + C[2][i2][d]
 * for run j' of row r with stage indices i0, i1, i2.
 *
 * moe_rvq_gemv: y[m][t][r] = sum_c W_m[r, c] x[t, c] for n_mats matrices at
 * mats + m * mat_stride (16-byte aligned; mat_stride a multiple of 16 and at
 * least one matrix when n_mats > 1), x bf16 or fp32 [T, K] (MOE_BF16 /
 * MOE_F32, 4-byte aligned), y fp32 [n_mats][T][R] (4-byte aligned), all
 * device memory; the per-group partial sums (fp32, summed over K groups of
 * 4 to 8 tiles in group order; the group size follows the shape and the
 * device's CU count, so results can differ in the last bits between devices)
 * live in the caller's workspace of moe_rvq_workspace_bytes (256-byte
 * aligned, sized for groups of 4 tiles); the tables are built in LDS.
 * Stream-ordered, no allocation, no host synchronisation; T = 0 is a no-op.
 * Errors: MOE_EINVAL (shapes, dtype, pointers, alignment), MOE_ENOMEM
 * (workspace too small), MOE_EHIP.  moe_rvq_workspace_bytes
 * returns 0 for an invalid shape (T outside 1..65535, K or R not a positive
 * multiple of 64, n_mats < 1, more than 2^31 outputs n_mats * T * R, or more
 * than 2^20 work items of 256 columns by 4096 rows). */
#define MOE_RVQ_TILE_BYTES 1536
uint64_t moe_rvq_workspace_bytes(int32_t n_tokens, int32_t k_cols, int32_t rows, int32_t n_mats);
int moe_rvq_gemv(const void *x, int32_t x_dtype, int32_t n_tokens, int32_t k_cols,
                 const void *mats, uint64_t mat_stride, int32_t n_mats, int32_t rows,
                 const void *codebooks, float *y, void *workspace, uint64_t workspace_bytes,
                 void *stream);

/* CRC-32 of n_bytes of device memory at dev_bytes (16-byte aligned), with
 * zlib's polynomial and conditioning (the record payload checksum), into
 * *crc_out (host).  Runs on the current device, ordered on `stream`, and
 * waits for the result; its partial results use the static scratch of
 * moe_forward_noalloc (calls that overlap one of those on the same GPU race).
 * n_bytes 0 gives 0 without touching the device.  Errors: MOE_EINVAL (null
 * pointer, misaligned address), MOE_EHIP. */
int moe_crc32(const void *dev_bytes, uint64_t n_bytes, uint32_t *crc_out, void *stream);

/* Test hook: dequantize a tiled matrix (bits 4 or 8) to fp32 [rows, cols] on
 * the GPU with the same decoding the kernels use. */
int moe_debug_dequant(const void *tiles, int32_t bits, int32_t rows, int32_t cols,
                      float *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QREB_MOE_H */
