/*
 * gdn.h -- C ABI of the Gated DeltaNet record / replay / GQA-expand library
 * (and the RMSNorm that precedes the layer) for AMD Instinct MI355X (gfx950).
 * Link with libgdn.so.
 *
 * Plain C: callers need neither HIP nor PyTorch headers.  Device pointers are
 * HIP device allocations; `stream` is a hipStream_t passed as void* (NULL is
 * the default stream).
 *
 * Common conventions
 * ------------------
 * - Layouts are dense and row-major with no strides (the index arithmetic of
 *   the record and replay kernels on the metaltile-std 0.1.0 page
 *   src/ffai/gated_delta_replay.rs, and its "Tape layout" paragraph):
 *       q, k            [B, T, Hk, Dk]      I/O dtype
 *       v, y, delta_log [B, T, Hv, Dv]      I/O dtype
 *       g, beta         [B, T, Hv]          I/O dtype
 *       k_log           [B, T, Hv, Dk]      I/O dtype (keys expanded to value heads)
 *       g_log           [B, T, Hv]          I/O dtype
 *       state           [B, Hv, Dv, Dk]     float32 always (row dv, column dk)
 *       mask            [B, T]              uint32; step active iff entry > 0
 * - Arithmetic is float32 throughout; every I/O element is widened to float32
 *   on load and rounded to nearest even on store.
 * - Ownership: the caller owns every buffer.  The library allocates nothing,
 *   keeps no state between calls and never synchronises; each call enqueues
 *   its kernel on `stream` and returns.  Ordering between calls is stream
 *   order.  Errors a kernel meets at run time (e.g. a fault) surface at the
 *   caller's next synchronisation, as usual in HIP.
 * - Validation happens on the host before any HIP call; a rejected call
 *   enqueues nothing and returns a negative gdn_status.  gdn_last_error()
 *   then holds a human-readable reason (per calling thread).
 * - Pointers to tensors other than mask, g, beta and g_log must be 16-byte
 *   aligned (mask 4-byte, the others element-aligned); gqa_expand needs only
 *   element alignment.
 * - Raw pointers carry no length: the caller guarantees each buffer holds the
 *   elements its shape implies.
 */
#ifndef GDN_H
#define GDN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 6

typedef enum gdn_dtype {
    GDN_F32 = 0,
    GDN_F16 = 1,
    GDN_BF16 = 2
} gdn_dtype;

typedef enum gdn_gqa_map {
    GDN_GQA_BLOCK = 0,  /* hk = hv / (Hv / Hk): consecutive value heads share a key head */
    GDN_GQA_TILED = 1   /* hk = hv mod Hk: the key heads repeat as a whole            */
} gdn_gqa_map;

typedef enum gdn_status {
    GDN_OK = 0,
    GDN_ERR_NULL = -1,              /* a required pointer is NULL                          */
    GDN_ERR_ZERO_DIM = -2,          /* a dimension is zero                                 */
    GDN_ERR_GQA_RATIO = -3,         /* Hk does not divide Hv (hg does not divide h)        */
    GDN_ERR_UNSUPPORTED_SHAPE = -4, /* (Dk, Dv) not built: see gdn_record                  */
    GDN_ERR_OVERFLOW = -5,          /* an element count or the launch grid is too large    */
    GDN_ERR_ALIAS = -6,             /* an output overlaps an input or another output       */
    GDN_ERR_BAD_ENUM = -7,          /* unknown dtype or GQA map                            */
    GDN_ERR_LAUNCH = -8,            /* the HIP runtime refused the launch                  */
    GDN_ERR_MISALIGNED = -9,        /* a pointer lacks the alignment stated above          */
    GDN_ERR_WORKSPACE = -10         /* workspace NULL or smaller than the call needs       */
} gdn_status;

/*
 * gdn_record -- gated delta-rule forward step with innovation-tape capture.
 *
 * Defined by the record kernel (macro `gated_delta_record!`) on the
 * metaltile-std 0.1.0 page src/ffai/gated_delta_replay.rs.  For every batch
 * row b, value head hv (key head hk given by `gqa_map`), value row dv and step
 * t = 0..T-1 whose mask entry is non-zero (all steps when mask == NULL):
 *     S[dv,:] <- g[b,t,hv] * S[dv,:]
 *     kv      <- S[dv,:] . k[b,t,hk,:]
 *     delta   <- (v[b,t,hv,dv] - kv) * beta[b,t,hv]
 *     delta_log[b,t,hv,dv] <- delta
 *     S[dv,:] <- S[dv,:] + delta * k[b,t,hk,:]
 *     y[b,t,hv,dv] <- S[dv,:] . q[b,t,hk,:]
 * starting from S = state_in[b,hv] and ending with state_out[b,hv] = S.
 * An inactive step changes nothing and writes nothing: y and delta_log keep
 * whatever the caller's buffers held at those positions.
 *
 * Optionally the call also captures the rest of the innovation tape that the
 * module documentation ("Tape layout") lists next to delta_log: at every
 * active step, k_log[b,t,hv,:] <- k[b,t,hk,:] (the keys expanded to value
 * heads under gqa_map) and g_log[b,t,hv] <- g[b,t,hv], both as bit copies.
 * gdn_replay then takes (delta_log, k_log, g_log) with no separate pass.
 *
 * Arguments
 *   q, k, v, g, beta  inputs, io_dtype, layouts above.
 *   state_in          float32 [B,Hv,Dv,Dk].
 *   mask              uint32 [B,T] or NULL (every step active).
 *   y                 output, io_dtype [B,T,Hv,Dv].
 *   state_out         output, float32 [B,Hv,Dv,Dk]; may be exactly state_in
 *                     (in place), but must not overlap it otherwise.
 *   delta_log         output tape, io_dtype [B,T,Hv,Dv], or NULL for the plain
 *                     forward step without a tape.
 *   k_log             optional output, io_dtype [B,T,Hv,Dk], or NULL.
 *   g_log             optional output, io_dtype [B,T,Hv], or NULL.
 *   B, T, Hk, Hv, Dk, Dv  sizes; Hk must divide Hv.  Dk in {32,64,128,192,256};
 *                     Dv a multiple of 16, at most 1024.  One launch covers
 *                     all B*Hv*Dv state rows with at most 2^32 - 1 threads
 *                     (16 per row, fewer with several rows per thread);
 *                     past that the call fails with GDN_ERR_OVERFLOW (split
 *                     the batch).
 *   io_dtype          gdn_dtype of every non-state tensor.
 *   gqa_map           gdn_gqa_map.
 *   stream            hipStream_t or NULL.
 * Returns GDN_OK or a negative gdn_status (nothing is enqueued on error).
 */
int gdn_record(const void* q, const void* k, const void* v, const void* g, const void* beta,
               const float* state_in, const uint32_t* mask,
               void* y, float* state_out, void* delta_log, void* k_log, void* g_log,
               uint32_t B, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dk, uint32_t Dv,
               int io_dtype, int gqa_map, void* stream);

/*
 * gdn_replay -- speculative-decode rollback: starting again from the state
 * saved before gdn_record ran, apply only the tape positions that were
 * accepted.
 *
 * Defined by the replay kernel (macro `state_replay!`) and the module
 * documentation ("Two kernels", "Tape layout") on the metaltile-std 0.1.0 page
 * src/ffai/gated_delta_replay.rs.  For every (b, hv, dv), starting from
 * S = state_in[b,hv], for t = 0..T_log-1 the step is taken iff t < accepted and
 * mask[b,t] > 0 (mask == NULL: every step passes); a taken step does
 *     S[dv,:] <- S[dv,:] * g_log[b,t,hv] + k_log[b,t,hv,:] * delta_log[b,t,hv,dv]
 * and an untaken one leaves S as it was, whatever its tape slot holds (NaN
 * included).  state_out[b,hv] = S.  accepted > T_log acts as T_log;
 * accepted == 0 copies the snapshot.
 *
 * Arguments
 *   delta_log   io_dtype [B,T_log,Hv,Dv].
 *   k_log       io_dtype [B,T_log,Hv,Dk] (keys already expanded to value heads,
 *               e.g. by gqa_expand).
 *   g_log       io_dtype [B,T_log,Hv].
 *   state_in    float32 [B,Hv,Dv,Dk], the snapshot taken before the record.
 *   mask        uint32 [B,T_log] or NULL.
 *   state_out   float32 [B,Hv,Dv,Dk]; may be exactly state_in.
 *   B, T_log, Hv, Dk, Dv, accepted   sizes and limits as for gdn_record.
 *   io_dtype, stream                 as for gdn_record.
 * Returns GDN_OK or a negative gdn_status.
 */
int gdn_replay(const void* delta_log, const void* k_log, const void* g_log,
               const float* state_in, const uint32_t* mask, float* state_out,
               uint32_t B, uint32_t T_log, uint32_t Hv, uint32_t Dk, uint32_t Dv,
               uint32_t accepted, int io_dtype, void* stream);

/*
 * gqa_expand -- GQA head broadcast [seq, hg, k] -> [seq, h, k], a bit copy.
 *
 * Defined on the mlx-native 0.6.5 page mlx_native/ops/repeat_tiled.rs (module
 * documentation "Mapping": dst[t,h,k] = src[t, h % hg, k], and the argument
 * rules of `dispatch_repeat_tiled_f32`), with the block map of the
 * metaltile-std record kernel as the alternative:
 *     GDN_GQA_TILED  dst[s,hh,e] = src[s, hh % hg,        e]
 *     GDN_GQA_BLOCK  dst[s,hh,e] = src[s, hh / (h / hg),  e]
 * Element bits are copied unchanged (NaN payloads included).  A batched
 * tensor [B,T,H,K] is expanded with seq = B*T.
 *
 * Arguments
 *   src, dst    device buffers of seq*hg*k and seq*h*k elements; must not
 *               overlap; element-aligned.
 *   seq, hg, h, k  sizes, all non-zero, hg dividing h.
 *   dtype       gdn_dtype (fixes the element size: 4 bytes for GDN_F32,
 *               2 for GDN_F16 and GDN_BF16).
 *   gqa_map     gdn_gqa_map.
 *   stream      hipStream_t or NULL.
 * Returns GDN_OK or a negative gdn_status.
 */
int gqa_expand(const void* src, void* dst, uint32_t seq, uint32_t hg, uint32_t h, uint32_t k,
               int dtype, int gqa_map, void* stream);

/*
 * gdn_prefill -- the record step of gdn_record over a long sequence (a
 * prefill), computed a chunk of 64 steps at a time on the matrix cores.
 *
 * Computes the same outputs as gdn_record with delta_log given (or NULL), from
 * the same definition: the record kernel (macro `gated_delta_record!`) on the
 * metaltile-std 0.1.0 page src/ffai/gated_delta_replay.rs.  The mlx-native
 * 0.6.5 page mlx_native/ops/repeat_tiled.rs names the "chunk-prefill" caller
 * that feeds it expanded keys; the chunk algorithm is this library's own: over
 * a chunk, the innovations solve a unit lower-triangular system in the chunk's
 * keys, gates and betas, and y and the state follow from matrix products.  The
 * arithmetic is reordered, so results agree with gdn_record to rounding (float32
 * accumulation; float32 operands enter the bf16 matrix cores as a sum of two
 * bf16 numbers, about 16 significant bits; fp16 keys and queries as an exact
 * sum of two bf16 numbers), not bit for bit.  Inactive steps (mask entry 0)
 * change nothing and write nothing, as in gdn_record.
 *
 * Arguments
 *   q .. g_log        as for gdn_record, including the optional tape capture:
 *                     k_log [B,T,Hv,Dk] receives at every active step the keys
 *                     expanded to value heads, g_log [B,T,Hv] the gates, both
 *                     as bit copies (NULL: not written).
 *   workspace         device scratch of at least gdn_prefill_workspace_size(B,
 *                     T, Hv) bytes, 256-byte aligned, owned by the caller and
 *                     overlapping no other argument.  Its contents on entry do
 *                     not matter; on return they are undefined.  Two calls in
 *                     flight at once need two workspaces.
 *   workspace_bytes   its size.
 *   B, T, Hk, Hv      sizes; Hk must divide Hv.
 *   Dk, Dv            Dk must be 128 or 192 (the page's shape-cell key
 *                     width), Dv a multiple of 16 up to 1024.
 *   io_dtype          GDN_BF16 or GDN_F16 (not GDN_F32).
 *   gqa_map, stream   as for gdn_record.
 * The call enqueues two kernels on `stream`.
 * Returns GDN_OK or a negative gdn_status (nothing is enqueued on error):
 * GDN_ERR_UNSUPPORTED_SHAPE for another dtype or head size, GDN_ERR_WORKSPACE
 * for a missing or short workspace.
 */
/* Bytes of workspace gdn_prefill needs for these sizes: 33280 per (batch row, value head, chunk
 * of 64 steps); UINT64_MAX if that does not fit in 64 bits. */
uint64_t gdn_prefill_workspace_size(uint32_t B, uint32_t T, uint32_t Hv);

int gdn_prefill(const void* q, const void* k, const void* v, const void* g, const void* beta,
                const float* state_in, const uint32_t* mask,
                void* y, float* state_out, void* delta_log, void* k_log, void* g_log,
                void* workspace, uint64_t workspace_bytes,
                uint32_t B, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                int io_dtype, int gqa_map, void* stream);

/*
 * gdn_prefill_noalloc -- gdn_prefill without a workspace argument, allocating
 * nothing.  For callers that cannot allocate device memory: code under HIP
 * graph capture, serving loops that must not allocate, harnesses that forbid
 * hipMalloc.
 *
 * Same arguments (less workspace and workspace_bytes), results and errors as
 * gdn_prefill; it runs the same kernels.  Its workspace is a scratch area of
 * GDN_PREFILL_SCRATCH_BYTES bytes inside the library: each GPU it runs on
 * holds its own copy from the first call until the process ends.  The call
 * allocates and frees nothing.  Sizes that need more (gdn_prefill_workspace_size
 * (B, T, Hv) > GDN_PREFILL_SCRATCH_BYTES, i.e. B * Hv * ceil(T / 64) > 2048,
 * e.g. past a 4096-step prefill over 32 value heads) fail with
 * GDN_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU uses
 * that one area, whose contents the previous call left: two calls whose
 * kernels overlap in time on one GPU (on different streams, or from threads
 * that do not order them) race and corrupt each other's results; calls
 * ordered on one stream are safe.  `stream` must belong to the current device
 * (GDN_ERR_LAUNCH otherwise).
 */
#define GDN_PREFILL_SCRATCH_BYTES 68157440ull

int gdn_prefill_noalloc(const void* q, const void* k, const void* v, const void* g, const void* beta,
                        const float* state_in, const uint32_t* mask,
                        void* y, float* state_out, void* delta_log, void* k_log, void* g_log,
                        uint32_t B, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                        int io_dtype, int gqa_map, void* stream);

/*
 * rms_norm_bf16 -- RMSNorm with bf16 weights over a batch of tokens.
 *
 * Defined on the moeflux 0.1.0-pre.3 page src/riir/backend/gpu/gpu_norm.rs
 * (documentation of `gpu_rms_norm_fused`, "GPU RMSNorm", and of the batched
 * `encode_rms_norm_bf16_fused_n_tokens`, one row per token): for every token t,
 *     out[t,i] = x[t,i] * (1 / sqrt(sum_i x[t,i]^2 / dim + eps)) * w[i],
 * w[i] the bf16 weight widened exactly.  Arithmetic is float32.
 *
 * Arguments
 *   x         float32 [n_tokens, dim], 4-byte aligned.
 *   weight    the bf16 weight [dim] as raw 16-bit patterns, 2-byte aligned.
 *   out       float32 [n_tokens, dim], 4-byte aligned; may be exactly x (in
 *             place), but must not overlap x otherwise, nor the weight.
 *   n_tokens, dim   sizes, non-zero.
 *   eps       added to the mean square (any value; the page passes a small
 *             positive constant).
 *   stream    hipStream_t or NULL.
 * The fastest path needs dim a multiple of 4 and at most 8192, x and out
 * 16-byte aligned and weight 8-byte aligned; other cases take a general path.
 * Returns GDN_OK or a negative gdn_status (nothing is enqueued on error).
 */
int rms_norm_bf16(const float* x, const uint16_t* weight, float* out, uint32_t n_tokens,
                  uint32_t dim, float eps, void* stream);

/*
 * Launch choices, for tests and launch-shape sweeps.
 *
 * gdn_record and gdn_replay pick their kernel and launch shape from the sizes
 * alone; nothing else (no environment, no state) changes what they run.
 * gdn_record_debug and gdn_replay_debug take the same arguments after a
 * gdn_launch_choice that forces those picks, so that tests can check every
 * kernel configuration against the others and sweeps can time each one.  A
 * NULL or all-zero choice leaves every pick to the library: the call is then
 * exactly gdn_record / gdn_replay.  Every configuration computes the same
 * function: row tilings change no bit of any output, and the two replay folds
 * agree within the stated tolerance (they round differently).
 *
 * Errors, besides those of the plain calls: a (rows_per_thread, threads) pair
 * that is not one of the five below, an unknown fold or a wave count other
 * than 0, 2 or 4 -> GDN_ERR_BAD_ENUM; a tiling whose rows per workgroup
 * (rows_per_thread * threads / 16) do not divide Dv, that would keep more than
 * 64 state values per lane (rows_per_thread * Dk / 16), or, for a record of
 * more than one step, covers more than 64 rows; or the matrix-core fold on a
 * float32 tape or with Dv not a multiple of 64 -> GDN_ERR_UNSUPPORTED_SHAPE.
 */
typedef enum gdn_replay_fold {
    GDN_FOLD_AUTO = 0,    /* the matrix cores for 16+ positions of a 16-bit tape with Dv % 64 == 0 */
    GDN_FOLD_VALU = 1,    /* the vector-ALU fold (any tape)                                        */
    GDN_FOLD_MATRIX = 2   /* the matrix-core fold (16-bit tape, Dv a multiple of 64)               */
} gdn_replay_fold;

typedef struct gdn_launch_choice {
    /* State rows per thread and threads per workgroup of the vector-ALU
     * kernels: (8,256), (4,256), (2,256), (1,256) or (1,64); both 0 for the
     * library's choice.  Ignored by a replay that runs on the matrix cores. */
    uint32_t rows_per_thread;
    uint32_t threads;
    int32_t replay_fold;      /* gdn_replay_fold; gdn_replay_debug only (0 for gdn_record_debug) */
    uint32_t matrix_waves;    /* matrix-core fold: waves per workgroup, 2 or 4; 0 for the library's (4) */
} gdn_launch_choice;

int gdn_record_debug(const gdn_launch_choice* choice,
                     const void* q, const void* k, const void* v, const void* g, const void* beta,
                     const float* state_in, const uint32_t* mask,
                     void* y, float* state_out, void* delta_log, void* k_log, void* g_log,
                     uint32_t B, uint32_t T, uint32_t Hk, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                     int io_dtype, int gqa_map, void* stream);

int gdn_replay_debug(const gdn_launch_choice* choice,
                     const void* delta_log, const void* k_log, const void* g_log,
                     const float* state_in, const uint32_t* mask, float* state_out,
                     uint32_t B, uint32_t T_log, uint32_t Hv, uint32_t Dk, uint32_t Dv,
                     uint32_t accepted, int io_dtype, void* stream);

/* Static description of a status code (never NULL). */
const char* gdn_strerror(int status);

/* Reason for the last failed call on this thread ("" if none yet). */
const char* gdn_last_error(void);

/* GDN_ABI_VERSION of the loaded library. */
int gdn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
