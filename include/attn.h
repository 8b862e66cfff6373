/*
 * attn.h -- C ABI of the exact-attention library for AMD Instinct MI355X
 * (gfx950).  Built as libattn.so; every entry point is extern "C" and takes
 * plain pointers and sizes.
 *
 * What is computed.  For every batch b and head h, with Q, K, V in R^{N x d}:
 *
 *   S = scale * Q K^T,  P = softmax(S) row by row,  O = P V,
 *   L_i = m_i + ln(l_i)  (the log-sum-exp of row i of the masked S),
 *
 * the standard-attention definition and the LSE statistic of the FLASH-ATTN
 * page (taking-lying-flat): "Background" of the FlashAttention summary for S,
 * P and O, and the FlashAttention-2 section for L = m + log(l) and the causal
 * mask (S_ij = -inf for j > i).  The N x N matrices S and P are never written
 * to memory: the forward streams K/V tiles through on-chip memory with the
 * online-softmax recurrence of that section and stores only O and L; the
 * backward rebuilds P tile by tile from L (the same page's "Tiling and
 * Recomputation").
 *
 * Masking (key j visible to query i):
 *   causal == 0, window == 0 : always
 *   causal == 1              : j <= i
 *   window == W > 0          : additionally |i - j| < W  (so with causal,
 *                              i - W < j <= i: the window counts the query's
 *                              own key).  W >= N with causal equals causal.
 * Every query sees at least its own key when causal or windowed, so no row of
 * P is empty.
 *
 * Shared key/value heads (multi-query and grouped-query attention, the
 * FLASH-ATTN page's FlashAttention-2 section): with H_kv > 0, the H query
 * heads of a batch element share H_kv key/value heads (H a multiple of
 * H_kv); query head h reads key/value head h / (H / H_kv), i.e. consecutive
 * query heads form a group.  Nothing is copied; the backward's dK and dV of
 * a shared head are the sums over its group.  H_kv = 0 (or H) is ordinary
 * multi-head attention, H_kv = 1 multi-query attention.
 *
 * Layouts.  Q, O, dO, dQ are dense [B][H][N][d] row-major (d fastest, no
 * padding); K, V, dK, dV are [B][H_kv][N][d] (H_kv = H when desc->H_kv is
 * 0); L and the backward workspace rows are [B][H][N].
 * bf16 is IEEE binary32 truncated to its upper 16 bits (round-to-nearest-even
 * when produced here).  fp8 inputs are OCP E4M3 ("fn": bias 7, max 448, no
 * infinities) with a per-tensor descale: value = code_value * descale.
 *
 * Ownership and streams.  Every tensor pointer is a device pointer allocated
 * by the caller; the library allocates nothing and keeps no state between
 * calls.  All work is enqueued on `stream` (a hipStream_t; NULL is the
 * default stream) and the call returns without waiting: faults in the
 * kernels surface at the caller's next synchronisation.  Outputs must not
 * alias inputs; outputs are overwritten, never accumulated into.
 *
 * Errors.  Arguments are checked on the host before anything is launched:
 *   ATTN_EINVAL        null required pointer, B/H/N < 1, window < 0, scale not
 *                      finite or <= 0, causal not 0/1, H_kv < 0 or H not a
 *                      multiple of H_kv, pointer not 16-byte aligned, output
 *                      dtype unknown, workspace too small;
 *   ATTN_EUNSUPPORTED  d not in {64, 128}, or B*H*N*d >= 2^31;
 *   ATTN_EHIP          the HIP runtime reported an error at launch.
 * On ATTN_EINVAL / ATTN_EUNSUPPORTED nothing has been enqueued.
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,
  ATTN_EUNSUPPORTED = 2,
  ATTN_EHIP = 3,
  ATTN_ESCRATCH = 4 /* attn_bwd_noalloc only: the problem exceeds its static scratch */
} attn_status;

typedef enum { ATTN_OUT_BF16 = 0, ATTN_OUT_F32 = 1 } attn_out_dtype;

typedef struct {
  int32_t B, H, N, d; /* batch, query heads, sequence length, head dim (64/128) */
  float scale;        /* s in softmax(s * Q K^T); finite and > 0                */
  int32_t causal;     /* 0 or 1                                                 */
  int32_t window;     /* 0 = no window; W > 0 as in the masking rule above      */
  int32_t H_kv;       /* key/value heads: 0 = H; else a divisor of H (above)    */
} attn_desc;

/* Forward, bf16 inputs (FLASH-ATTN page, FlashAttention-2 section: the
 * unnormalised accumulator O~ <- diag(e^{m_old - m_new}) O~ + e^{S - m_new} V,
 * divided by l once at the end).
 *   q       : bf16 [B,H,N,d];  k, v : bf16 [B,H_kv,N,d]
 *   o       : [B,H,N,d], bf16 (o_dtype = ATTN_OUT_BF16) or fp32 (ATTN_OUT_F32)
 *   lse     : fp32 [B,H,N], natural-log LSE of the scaled, masked scores;
 *             may be NULL when the caller does not need it.               */
attn_status attn_fwd(const attn_desc* desc, const void* q, const void* k,
                     const void* v, void* o, int32_t o_dtype, float* lse,
                     void* stream);

/* Bytes of device workspace the backward needs for `desc`: two fp32 [B,H,N]
 * arrays, D_i = sum_k dO_ik O_ik and L_i log2(e), each padded to a multiple
 * of 256 bytes; for grouped-query attention (H_kv < H) whose dK/dV pass would
 * otherwise run on too few workgroups (less than one round over the 256
 * CUs, a round being one workgroup per CU at d = 128 and two at d = 64; with
 * the causal mask, less than two rounds), also two fp32 arrays of
 * S x [B,H_kv,N,d] partial dK and dV, where the query heads of each group
 * are split into S shares (S a divisor of H / H_kv) whose sums are added by
 * a second launch in share order (deterministic).  Depends on B, H, H_kv, N,
 * d and causal.  0 if `desc` is invalid. */
size_t attn_bwd_workspace_bytes(const attn_desc* desc);

/* Backward (FLASH-ATTN page, FlashAttention-2 summary "Background": dV = P^T dO,
 * dP = dO V^T, dS = dsoftmax(dP), dQ = dS K, dK = dS^T Q; with the scale s
 * carried through, dQ = s dS K and dK = s dS^T Q, and dsoftmax written out as
 * dS_ij = P_ij (dP_ij - D_i), D_i = sum_k dO_ik O_ik).  P is recomputed from
 * Q, K and the forward's L; it is never read from memory.
 *   q, o, dout       : bf16 [B,H,N,d]  (o is the forward's bf16 output)
 *   k, v             : bf16 [B,H_kv,N,d]
 *   lse              : fp32 [B,H,N] from attn_fwd with the same desc
 *   dq               : fp32 [B,H,N,d], overwritten
 *   dk, dv           : fp32 [B,H_kv,N,d], overwritten (summed over groups)
 *   workspace        : device memory of at least attn_bwd_workspace_bytes */
attn_status attn_bwd(const attn_desc* desc, const void* q, const void* k,
                     const void* v, const void* o, const void* dout,
                     const float* lse, float* dq, float* dk, float* dv,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The backward for callers that cannot allocate memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): attn_bwd
 * without a workspace argument.  Its D and L log2(e) arrays live in a static
 * device array of the library, ATTN_NOALLOC_SCRATCH_BYTES bytes on every GPU
 * the library runs on, held until the process ends; the call allocates
 * nothing and calls no allocating routine.  The scratch holds
 * attn_bwd_noalloc_scratch_bytes(desc) bytes (8 bytes per query row, each
 * array padded to 256 bytes), so B*H*N may be at most about 2^21; larger
 * problems return ATTN_ESCRATCH before anything is launched.  Grouped-query
 * backwards never split a group here (no partial dK/dV arrays), so small
 * grouped-query grids may run slower than with attn_bwd.
 *   The scratch is shared by every call on a GPU and keeps the last call's
 * contents (each call writes all of what it reads first, so nothing needs
 * clearing); calls that overlap on one GPU (for example on two streams) race
 * on it and must be serialised by the caller.  The scratch's device address
 * is looked up once per device, on the first call with that device current;
 * `stream` must belong to the current device.  Other arguments, results and
 * errors as attn_bwd. */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
size_t attn_bwd_noalloc_scratch_bytes(const attn_desc* desc);
attn_status attn_bwd_noalloc(const attn_desc* desc, const void* q, const void* k,
                             const void* v, const void* o, const void* dout,
                             const float* lse, float* dq, float* dk, float* dv,
                             void* stream);

/* The backward as separately launchable stages.  attn_bwd enqueues
 * attn_bwd_dq and then attn_bwd_dkdv on one stream; a caller may issue them
 * itself (for example to time them).  Argument rules as attn_bwd.
 *   attn_bwd_dq:         dQ = s dS K, one pass per query block over the K/V
 *                        blocks it sees (S and dP are recomputed there).  It
 *                        forms D_i = sum_k dO_ik O_ik of its own rows and
 *                        also writes D and L log2(e) to the workspace.
 *   attn_bwd_dkdv:       dK = s dS^T Q and dV = P^T dO, one pass per K/V block
 *                        over the query blocks that see it (the FLASH-ATTN
 *                        page's column-block partition of the backward).  It
 *                        reads D and L log2(e) from the workspace, which
 *                        attn_bwd_dq or attn_bwd_preprocess must have filled
 *                        from the same o, dout and lse earlier on the stream.
 *   attn_bwd_preprocess: only fills the workspace (D and L log2(e)), for a
 *                        caller that runs attn_bwd_dkdv without attn_bwd_dq. */
attn_status attn_bwd_dq(const attn_desc* desc, const void* q, const void* k,
                        const void* v, const void* o, const void* dout,
                        const float* lse, void* workspace, size_t workspace_bytes,
                        float* dq, void* stream);
attn_status attn_bwd_dkdv(const attn_desc* desc, const void* q, const void* k,
                          const void* v, const void* dout, const void* workspace,
                          size_t workspace_bytes, float* dk, float* dv, void* stream);
attn_status attn_bwd_preprocess(const attn_desc* desc, const void* o,
                                const void* dout, const float* lse, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Forward with fp8 inputs (FLASH-ATTN page, FlashAttention-3 summary,
 * "Low-precision with FP8": E4M3 inputs with one scale per tensor).  q8
 * [B,H,N,d] and k8, v8 [B,H_kv,N,d] are E4M3 codes; the inputs are
 * code * descale.  Both products run on the 16-bit matrix cores: each tile
 * is widened in LDS, exactly, to bf16 (Q, K) or fp16 (V); the scores are
 * summed in fp32 and the probabilities enter the P V product as fp16.  (The
 * fp8 matrix instruction keeps too few bits of its 64-product sums for
 * inputs with outlier channels, and an fp8 P accurate enough for them needs
 * two E4M3 terms, i.e. as many matrix cycles as fp16.)  o and lse as in
 * attn_fwd. */
attn_status attn_fwd_fp8(const attn_desc* desc, const uint8_t* q8,
                         const uint8_t* k8, const uint8_t* v8, float q_descale,
                         float k_descale, float v_descale, void* o,
                         int32_t o_dtype, float* lse, void* stream);

/* The fp8 forward with one descale per block instead of per tensor (the
 * FLASH-ATTN page's FlashAttention-3 summary, block quantisation: Q, K, V cut
 * into row blocks that are quantised independently, the S tiles rescaled by
 * the blocks' factors at no extra cost).  Block sizes are this kernel's
 * tiles: 128 query rows, 64 key rows.
 *   q_descales : fp32 [B,H,ceil(N/128)]   (query block qb covers rows 128 qb ..)
 *   k_descales : fp32 [B,H_kv,ceil(N/64)] (key block kb covers rows 64 kb ..)
 *   v_descales : fp32 [B,H_kv,ceil(N/64)]
 * The real inputs are code * the descale of the code's block; every descale
 * must be finite and > 0, and every value descale below 255 (the fp16
 * probabilities carry it); device memory, so not checked.  Incoherent processing
 * (multiplying Q and K by one random orthogonal matrix before quantising,
 * same page) needs nothing from the kernel, since (QM)(KM)^T = QK^T: the
 * caller transforms and quantises.  Other arguments as attn_fwd_fp8. */
attn_status attn_fwd_fp8_blocks(const attn_desc* desc, const uint8_t* q8,
                                const uint8_t* k8, const uint8_t* v8,
                                const float* q_descales, const float* k_descales,
                                const float* v_descales, void* o, int32_t o_dtype,
                                float* lse, void* stream);

/* A short block of queries against a long key/value sequence (decode): the
 * N_q queries of each head are the last N_q positions of a sequence of N_k
 * keys, so query row i sits at key position N_k - N_q + i and the masks above
 * apply to that position (causal: key j visible iff j <= N_k - N_q + i; the
 * pages fix no alignment for N_q < N_k, and this one gives attn_fwd's rows
 * when N_q = N_k).  Decode is bound by reading K and V once (FlashAttention-3
 * page, the point on inference), so the keys are split into chunks that run
 * in parallel, each giving a partial (O_c, L_c) per query row, and a second
 * launch merges them with the softmax decomposition of the FLASH-ATTN page
 * ("Tiling and Recomputation"): L = ln sum_c e^{L_c}, O = sum_c e^{L_c - L} O_c.
 *   q        : bf16 [B,H,N_q,d];  k, v : bf16 [B,H_kv,N_k,d] (H_kv = 0 means H)
 *   o, lse   : as attn_fwd, [B,H,N_q,d] and [B,H,N_q] (lse may be NULL)
 *   workspace: device memory of at least attn_decode_workspace_bytes(desc)
 *              bytes (the partials); its contents on entry do not matter.
 * Errors as above, and ATTN_EINVAL when N_q < 1 or N_q > N_k. */
typedef struct {
  int32_t B, H, H_kv; /* batch, query heads, key/value heads (0 = H)        */
  int32_t N_q, N_k, d; /* queries per head, keys per head, head dim (64/128) */
  float scale;        /* s in softmax(s * Q K^T); finite and > 0             */
  int32_t causal;     /* 0 or 1                                              */
  int32_t window;     /* 0 = no window; W > 0 as in the masking rule above   */
} attn_decode_desc;

size_t attn_decode_workspace_bytes(const attn_decode_desc* desc);
attn_status attn_fwd_decode(const attn_decode_desc* desc, const void* q, const void* k,
                            const void* v, void* o, int32_t o_dtype, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Dropout on the probabilities (the FLASH-ATTN page lists dropout among the
 * variants the fused kernel supports, and its FlashAttention-2 "Background"
 * paragraph names dropout on P as one of the elementwise steps that the fused
 * kernel keeps on chip).  The pages fix no random-number contract; this is
 * the library's:
 *   t       = round(256 p), halves up (t = floor(256 p + 1/2), in double);
 *   byte    = byte (j mod 4) (least significant first) of word (i mod 4) of
 *             Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) with counter
 *             (floor(j/4), floor(i/4), bh, offset) and key (seed mod 2^32,
 *             floor(seed / 2^32)), for query head bh = b * H + h, query i and
 *             key j of that head;
 *   Z_ij    = 1 if byte >= t, else 0 (keep probability q = (256 - t) / 256);
 *   O       = (P o Z / q) V, with P the softmax of the masked scores, and lse
 *             the log-sum-exp of those scores (dropout does not change it).
 * The backward uses the same Z: dV = (P o Z / q)^T dO, dP = (dO V^T) o Z / q,
 * dS = P o (dP - D) with D_i = sum_k dO_ik O_ik of the dropped O, dQ = s dS K,
 * dK = s dS^T Q.  p = 0 runs the ordinary kernels. */
typedef struct {
  float p;            /* dropout probability: 0 <= p and round(256 p) <= 255 */
  uint32_t offset;    /* fourth counter word (e.g. a step number)            */
  uint64_t seed;      /* Philox key                                          */
} attn_dropout;

/* attn_fwd with dropout on P (bf16 inputs; o, lse as attn_fwd).  ATTN_EINVAL
 * also for a NULL `drop`, p not finite, p < 0 or round(256 p) > 255. */
attn_status attn_fwd_dropout(const attn_desc* desc, const attn_dropout* drop,
                             const void* q, const void* k, const void* v, void* o,
                             int32_t o_dtype, float* lse, void* stream);

/* attn_bwd of attn_fwd_dropout: the same desc and drop (p, offset, seed) as
 * the forward that produced o and lse; other arguments and errors as attn_bwd
 * and attn_fwd_dropout.  Enqueues the dQ pass, then the dK/dV pass. */
attn_status attn_bwd_dropout(const attn_desc* desc, const attn_dropout* drop,
                             const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, float* dq, float* dk,
                             float* dv, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Which kernel an entry point runs (for matching profiler traces).  Returns
 * the symbol of the main kernel -- the one that does the attention
 * arithmetic -- that the entry point of `stage` launches for `desc`, as
 * profilers list it (for example "attn::fwd_pp_kernel<128, 4, 32>"):
 *   ATTN_STAGE_FWD      attn_fwd (dropout_p = 0) or attn_fwd_dropout
 *   ATTN_STAGE_BWD_DQ   attn_bwd_dq, the dQ pass of attn_bwd / attn_bwd_dropout
 *   ATTN_STAGE_BWD_DKDV attn_bwd_dkdv, the dK/dV pass of the same
 *   ATTN_STAGE_FWD_FP8  attn_fwd_fp8 (dropout_p must be 0)
 * Nothing is launched.  Static storage, valid until the process ends; NULL
 * for an invalid desc, stage or dropout_p (rules as the entry points). */
typedef enum {
  ATTN_STAGE_FWD = 0,
  ATTN_STAGE_BWD_DQ = 1,
  ATTN_STAGE_BWD_DKDV = 2,
  ATTN_STAGE_FWD_FP8 = 3
} attn_stage;
const char* attn_kernel_name(const attn_desc* desc, int32_t stage, float dropout_p);

/* Static, human-readable text for a status code. */
const char* attn_status_str(attn_status status);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */
