/*
 * libloopvq -- LoopVQ sub-bit KV-cache decode attention and encoder for
 * AMD Instinct MI355X (gfx950).  C ABI; plain pointers and sizes.
 *
 * What it computes (the LoopVQ pages):
 *  - LoopVQ project page (mscheong01.github.io/loopvq), "Method" and the
 *    "Overview of LoopVQ" figure: the keys and values of a looped model are
 *    vector-quantised with sub-vectors that span G/Tc channels at each of Tc
 *    consecutive loop steps, so a single 8-bit index serves all Tc steps;
 *    at loop step t the index is read through slice t of the codeword.
 *  - same page, "Serving in SGLang": new keys/values are written in bf16
 *    ("Write in bf16"); the first n_sink and the most recent n_recent tokens
 *    stay bf16 at every loop step; older tokens are encoded into shared
 *    indices ("Encode in pages"); at step t attention reads the keys and
 *    values from the indices through codebook slice t and merges with the
 *    bf16 attention over the sink and recent tokens ("Attend from indices").
 *  - same page, "Results -- Long-context retrieval": n_sink = 64 and
 *    n_recent = 256.
 *
 * Notation: B sequences, H query heads, Hk KV heads (Hk = H for multi-head
 * attention; Hk dividing H for grouped-query attention, where query head h
 * reads KV head h / (H / Hk)), d = head_dim, Tc = loop_steps (loop steps
 * sharing one index), R = n_loops (loop steps of the model, a multiple of Tc;
 * R = Tc unless set), G = group (elements per sub-vector), cg = G / Tc
 * channels per loop step, S = d / cg sub-vectors per token per head, 256
 * codes.  bits per cached element = 8 / G.  With R > Tc a token keeps R / Tc
 * index rows: group g serves loop steps g*Tc .. g*Tc + Tc - 1 through
 * codebook slices g*Tc + t.
 *
 * Storage layouts (all row-major, innermost last):
 *   x (encoder input) bf16  [n_tokens][Hk][R][d]  (or strided, see lvq_encode)
 *   codebook          f32 or bf16 [R][Hk][256][S][cg]: entry i = t*cg + c of
 *                     codeword k of (group g, head h, sub-vector j) at
 *                     [g*Tc + t][h][k][j][c]: slice r of a head is contiguous,
 *                     and its row k holds code k of every sub-vector (the
 *                     table row a decode gather reads)
 *   index cache       uint8 [B][Hk][max_tokens][S] (R = Tc), or
 *                     [R/Tc][B][Hk][max_tokens][S] (one such block per group);
 *                     row p holds token p (absolute position); rows of bf16
 *                     tokens are unused
 *   window buffers    bf16 [B][R][Hk][n_sink + n_recent][d]: sink token p
 *                     (p < n_sink) in slot p; recent token p (p >= n_sink) in
 *                     slot n_sink + ((p - n_sink) mod n_recent)  (a ring)
 *   query             bf16 [B][H][d] (the query of the loop step decoded)
 *   output            fp32 [B][H][d]
 *
 * Windows of a context of L tokens (L counts the current token):
 *   sink   = [0, n_s),        n_s = min(L, n_sink)
 *   VQ     = [n_s, n_s + n_v), n_v = vq_len[b] if given, else
 *                              max(0, L - n_sink - n_recent)
 *   recent = [n_s + n_v, L)
 *
 * Ownership and threading: the caller allocates and owns every buffer (device
 * memory unless stated).  The library never allocates, never synchronises the
 * host, keeps no global state and never prints.  Calls are asynchronous on the
 * given HIP stream (NULL = the default stream).  Concurrent calls must use
 * distinct workspaces.
 */
#ifndef LOOPVQ_H
#define LOOPVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LVQ_OK = 0,
    LVQ_ERR_INVALID_ARG = 1,  /* null pointer, inconsistent shape, bad index */
    LVQ_ERR_UNSUPPORTED = 2,  /* valid shape the kernels are not built for    */
    LVQ_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required   */
    LVQ_ERR_HIP = 4           /* a HIP launch reported an error               */
} lvq_status;

typedef enum { LVQ_F32 = 0, LVQ_BF16 = 1 } lvq_dtype;

typedef struct {
    int32_t batch;          /* B, >= 1                                        */
    int32_t n_heads;        /* H, >= 1                                        */
    int32_t head_dim;       /* d                                              */
    int32_t loop_steps;     /* Tc, divides group                              */
    int32_t group;          /* G; cg = G/Tc must divide d                     */
    int32_t n_sink;         /* bf16 sink tokens, >= 0 (64 on the pages)       */
    int32_t n_recent;       /* bf16 recent tokens, >= 1 (256 on the pages);
                               n_sink + n_recent <= LVQ_MAX_WINDOW_SLOTS    */
    int32_t max_tokens;     /* rows of the index cache per (b, h)             */
    int32_t codebook_dtype; /* lvq_dtype                                      */
    int32_t decode_splits;  /* workgroups per (b, h) for lvq_decode_attn;
                               0 = chosen by the library; 1..LVQ_MAX_SPLITS.
                               Changes only the rounding of the result.        */
    int32_t n_kv_heads;     /* Hk: heads of the index caches, codebooks and
                               windows; 0 = n_heads (multi-head attention);
                               otherwise must divide n_heads (grouped-query
                               attention, consecutive query heads sharing a
                               KV head)                                        */
    int32_t n_loops;        /* R: loop steps of the model; 0 = loop_steps;
                               otherwise a multiple of loop_steps, at most
                               LVQ_MAX_LOOPS                                   */
    int32_t decode_window_groups; /* with decode_splits = n > 1 on a grid of
                               at most 256 workgroups: how many of the n split
                               the bf16 window slots (the others take VQ
                               chunks); 0 = 1; otherwise 1..min(n - 1,
                               LVQ_MAX_WINDOW_GROUPS).  Must be 0 when
                               decode_splits is 0.  Changes only the rounding
                               of the result.                                   */
    int32_t decode_poll_limit; /* >= 0: how many times the workgroup that merges
                               the split partials of a (b, h) polls for them
                               before it gives up (writes NaN for that row and
                               sets LVQ_STATUS_MERGE_TIMEOUT); 0 = the default,
                               2^22 polls (seconds)                              */
    int32_t decode_heads_per_group; /* query heads per decode workgroup.  With
                               grouped-query attention two consecutive query
                               heads of one KV head can share a workgroup,
                               which reads each index row and window row once
                               for both.  0 = the library's choice: 2 where
                               possible (n_heads / n_kv_heads even, S = 32,
                               cg = 4, bf16 codebooks, head_dim 128, one layer
                               per launch, and a plan that merges through
                               window workgroups or needs no merge), else 1;
                               1 = one head; 2 = two (lvq_decode_attn returns
                               LVQ_ERR_UNSUPPORTED where not possible).  With
                               two heads, decode_splits counts workgroups per
                               (b, head pair).  Changes only the rounding of
                               the result.                                       */
} lvq_config;

#define LVQ_MAX_SPLITS 64
#define LVQ_MAX_WINDOW_GROUPS 4
#define LVQ_MAX_WINDOW_SLOTS (1 << 24)
#define LVQ_MAX_LOOPS 64
#define LVQ_MAX_LAYERS 4096
#define LVQ_CODES 256

/* Flags of the workspace status word (lvq_decode_status). */
#define LVQ_STATUS_MERGE_TIMEOUT 1u /* a merge gave up waiting for a split
                                       partial: that (b, h) row of out holds
                                       NaN; zero-fill the workspace before
                                       its next use                          */
#define LVQ_STATUS_VALUE_RANGE 2u   /* a bf16 value codebook entry read by a
                                       decode lies outside fp16's finite range
                                       (|v| >= 65536, or not finite): the value
                                       sums clamped it                       */

typedef struct {
    int32_t ndim;
    int64_t shape[6];
    int64_t stride[6];      /* in elements                                    */
    uint64_t bytes;
} lvq_tensor;

typedef struct {
    int32_t n_sub;                     /* S                                   */
    int32_t sub_channels;              /* cg                                  */
    int32_t n_codes;                   /* 256                                 */
    int32_t window_slots;              /* n_sink + n_recent                   */
    double bits_per_element;           /* 8 / G                               */
    double compression_vs_bf16;        /* 16 / bits_per_element               */
    double read_reduction_per_step;    /* bf16 K+V bytes per token and loop
                                          step / index bytes read per token and
                                          loop step = 2G/Tc                    */
    lvq_tensor k_index, v_index;       /* uint8                               */
    lvq_tensor k_codebook, v_codebook; /* codebook_dtype                      */
    lvq_tensor k_window, v_window;     /* bf16                                */
    lvq_tensor query;                  /* bf16                                */
    lvq_tensor output;                 /* fp32                                */
    uint64_t workspace_bytes;          /* for lvq_decode_attn                 */
} lvq_layout;

/*
 * Sizes and strides of every buffer for a configuration (pure host
 * arithmetic; no device is touched).  The bits-per-element and read-reduction
 * figures are the quantities the project page reports ("Highlights";
 * "Efficiency -- Latency").
 * Errors: LVQ_ERR_INVALID_ARG for a null pointer or an inconsistent config.
 */
lvq_status lvq_cache_layout(const lvq_config *cfg, lvq_layout *out);

/*
 * Encoder: nearest codeword of every loop-stacked sub-vector (LoopVQ project
 * page, "Component 1 -- Loop-axis vector quantization" and "Serving in SGLang
 * -- Encode in pages"; the news article "How LoopVQ works").
 *
 * Sub-vector j of (token n, head h, group g) has entries
 * x_i = x[n][h][g*Tc + t][j*cg + c], i = t*cg + c, and is coded with the
 * codewords of group g.  Its code is the k minimising the squared distance
 * D_k = sum_i (x_i - c_{k,i})^2 evaluated in IEEE fp32 (separate subtract,
 * square and add, ascending i); the lowest k wins ties.  The result is
 * bit-identical to that definition: the kernel screens all 256 codes with a
 * bf16 MFMA contraction and re-scores exactly every sub-vector whose two best
 * screen values lie within the screen's error bound (runs of up to 32 tokens
 * evaluate every distance directly).
 *
 * x          device bf16; element (n, h, t, ch) at
 *            x[n*x_strides[0] + h*x_strides[1] + t*x_strides[2] + ch];
 *            x_strides == NULL means the dense [n_tokens][Hk][R][d] layout
 *            (the KV heads, every loop step of the model; all R / Tc groups
 *            are encoded).
 *            Strides are in elements; channels must be contiguous and every
 *            stride a multiple of cg.
 * codebook   device, cfg->codebook_dtype, layout above, 16-byte aligned (one
 *            call encodes one tensor: call once with the K codebook and once
 *            with the V one); entries finite and below 2^127 in magnitude
 *            (the screen holds -2c)
 * index_cache device uint8 [B][Hk][max_tokens][S], 4-byte aligned; rows
 *            [first_token, first_token + n_tokens) of sequence seq are written
 * n_tokens   may be 0 (nothing launched)
 * Errors: LVQ_ERR_INVALID_ARG (null pointers, misaligned x, codebook or index_cache, seq
 * or rows out of range, bad strides), LVQ_ERR_UNSUPPORTED (G not in
 * {8, 16, 32}, cg not in {2, 4, 8}, S = d/cg not a multiple of 4, or fp32
 * codebooks with G = 32), LVQ_ERR_HIP.
 */
lvq_status lvq_encode(const lvq_config *cfg, const void *x, const int64_t *x_strides,
                      int64_t n_tokens, const void *codebook, uint8_t *index_cache,
                      int32_t seq, int64_t first_token, void *stream);

/*
 * The K and V of one run of tokens in a single launch (LoopVQ project page,
 * "Serving in SGLang -- Encode in pages": every page evicted from the recent
 * window is encoded into the K and the V index caches).  Identical to
 * lvq_encode(k_x, k_codebook, k_index) followed by lvq_encode(v_x,
 * v_codebook, v_index) with the same cfg, x_strides, n_tokens, seq and
 * first_token, but both tensors are encoded by one kernel launch (per group
 * of Tc loop steps), so a page costs one launch instead of two.  Arguments,
 * layouts, alignment and errors as for lvq_encode; nothing is launched unless
 * both tensors' arguments are valid.
 */
lvq_status lvq_encode_kv(const lvq_config *cfg, const void *k_x, const void *v_x,
                         const int64_t *x_strides, int64_t n_tokens, const void *k_codebook,
                         const void *v_codebook, uint8_t *k_index, uint8_t *v_index,
                         int32_t seq, int64_t first_token, void *stream);

/*
 * Decode attention of loop step r in [0, R) (LoopVQ project page, "Serving in
 * SGLang -- Attend from indices"): for every (b, h),
 *   out = sum_n softmax_n(sm_scale * q . K_n) V_n
 * over all L_b tokens, where VQ tokens use K_n[j*cg + c] =
 * k_codebook[r][h][k_index[g][b][h][n][j]][j][c] with g = r / Tc (likewise V;
 * g is absent when R = Tc) and sink/recent tokens use the bf16 window buffers
 * of step r.  fp32 accumulation; VQ value
 * rows enter as fp16 (exact for bf16 codebook entries of magnitude in
 * [2^-14, 65504], truncated toward zero below, by less than 2^-24; larger
 * entries are outside the supported range) weighted by fp16-rounded softmax
 * weights (relative 2^-11).
 * With grouped-query attention (n_kv_heads < n_heads) query head h reads the
 * caches, codebooks and windows of KV head h / (n_heads / n_kv_heads) with
 * its own query.  One kernel launch on `stream`; one workgroup of every
 * (b, h) merges the split partials.  Results depend on the split count only through
 * rounding.
 *
 * q          device bf16 [B][H][d], 16-byte aligned
 * ctx_len    device int32 [B]: L_b, precondition 0 <= L_b <= max_tokens
 *            (clamped on the device; L_b = 0 writes zeros)
 * vq_len     device int32 [B] or NULL (exact windows).  Precondition
 *            L_b - n_s - n_recent <= vq_len[b] <= L_b - n_s (clamped on the
 *            device; a recent window longer than n_recent keeps only the
 *            newest n_recent tokens).
 * max_ctx_len host int32: an upper bound of every L_b; sizes the launch.
 * k_codebook, v_codebook  16-byte aligned.
 * workspace  device, >= layout.workspace_bytes, 256-byte aligned; zero-filled
 *            once after allocation; every completed call leaves it valid for
 *            the next, whatever batch, head count, layer count or head_dim
 *            the next call has (as long as it is large enough for it): a
 *            status word, then per (layer, b, h) a block on a fixed grid
 *            holding an arrival word (a call epoch) and split partials
 *            tagged with that epoch.  Calls that share a workspace must not
 *            overlap in time (one stream, or ordered streams).
 * out        device fp32 [B][H][d]
 * Errors: LVQ_ERR_INVALID_ARG (null pointers, misaligned buffers, loop_step
 * outside [0, R), max_tokens < 1, max_ctx_len outside [0, max_tokens],
 * sm_scale not finite), LVQ_ERR_UNSUPPORTED (S = d/cg not in {8, 16, 32, 64},
 * cg not in {2, 4, 8}, a value-table row (S*cg entries of 2 bytes for bf16,
 * 4 for fp32 codebooks) above 256 bytes: e.g. d = 256 at G = 16, or
 * max_tokens * S near 2^31), LVQ_ERR_WORKSPACE, LVQ_ERR_HIP.
 */
lvq_status lvq_decode_attn(const lvq_config *cfg, int32_t loop_step, const void *q,
                           const int32_t *ctx_len, const int32_t *vq_len,
                           int32_t max_ctx_len, const uint8_t *k_index,
                           const uint8_t *v_index, const void *k_codebook,
                           const void *v_codebook, const void *k_window,
                           const void *v_window, float sm_scale, void *workspace,
                           uint64_t workspace_bytes, float *out, void *stream);

/*
 * lvq_decode_attn for callers that cannot allocate device memory at all (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, with no workspace argument.
 * The split partials live in a static device array of the library
 * (LVQ_NOALLOC_SCRATCH_BYTES per device, zero at load and kept until the
 * process ends; its address is looked up with hipGetSymbolAddress on a
 * device's first call, which allocates nothing).  The call itself calls no
 * allocating routine.
 *
 * Limit: a call whose plan merges split partials (more than one workgroup
 * per (b, h), e.g. long contexts at small batch) may cover at most
 * LVQ_NOALLOC_MAX_HEADS (b, h) pairs; larger ones return LVQ_ERR_WORKSPACE
 * before anything is launched.  Calls with one workgroup per (b, h) (e.g. a
 * batch of 64 sequences of 16 heads) have no limit.
 * Every call on a device shares that device's array: calls that overlap in
 * time on one device (other streams, other threads) race and must not be
 * made.  The status flags these calls set are kept in the array and cannot
 * be read; a merge that timed out shows as a NaN row of out, after which
 * later merging calls on that device may be wrong (the array cannot be
 * cleared): use lvq_decode_attn with a workspace of your own then.
 * Arguments, results and other errors as for lvq_decode_attn.
 */
#define LVQ_NOALLOC_MAX_HEADS 256
#define LVQ_NOALLOC_SCRATCH_BYTES 17105152u
lvq_status lvq_decode_attn_noalloc(const lvq_config *cfg, int32_t loop_step, const void *q,
                                   const int32_t *ctx_len, const int32_t *vq_len,
                                   int32_t max_ctx_len, const uint8_t *k_index,
                                   const uint8_t *v_index, const void *k_codebook,
                                   const void *v_codebook, const void *k_window,
                                   const void *v_window, float sm_scale, float *out,
                                   void *stream);

/* The operands of one layer of lvq_decode_attn_layers: the device buffers
 * that lvq_decode_attn takes, with the same layouts and alignments. */
typedef struct {
    const void *q;              /* bf16 [B][H][d]                               */
    const uint8_t *k_index;     /* index caches of the layer                    */
    const uint8_t *v_index;
    const void *k_codebook;     /* codebooks of the layer                       */
    const void *v_codebook;
    const void *k_window;       /* bf16 window buffers of the layer             */
    const void *v_window;
    float *out;                 /* fp32 [B][H][d]                               */
} lvq_decode_layer;

/* lvq_decode_attn for n_layers layers that share the config, the sequence
 * lengths and the loop step (several layers' caches attended at once, e.g.
 * independent requests that reach the same step; one launch per 16 layers,
 * so the launch and the split merge are paid once for all of them).  Each
 * layer computes exactly what lvq_decode_attn computes for its buffers (the
 * operation of the LoopVQ project page, "Serving in SGLang -- Attend from
 * indices"); results differ from separate calls only by rounding, through
 * the split count.
 *
 * layers     host array [n_layers], 1 <= n_layers <= LVQ_MAX_LAYERS; every
 *            pointer as for lvq_decode_attn.
 * workspace  device, >= n_layers * layout.workspace_bytes, 256-byte aligned,
 *            zero-filled once after allocation; the status word is shared and
 *            layer l uses the blocks of (l * B + b) * H + h, so layer 0 uses
 *            exactly the blocks of lvq_decode_attn and the two may share one
 *            workspace.
 * Other arguments and errors as for lvq_decode_attn (LVQ_ERR_INVALID_ARG also
 * for n_layers outside [1, LVQ_MAX_LAYERS] or a null layers array).
 */
lvq_status lvq_decode_attn_layers(const lvq_config *cfg, int32_t n_layers, int32_t loop_step,
                                  const lvq_decode_layer *layers, const int32_t *ctx_len,
                                  const int32_t *vq_len, int32_t max_ctx_len, float sm_scale,
                                  void *workspace, uint64_t workspace_bytes, void *stream);

/* Status flags that decode calls have set in a workspace (LVQ_STATUS_*; 0
 * when every call completed normally), for callers that check for a merge
 * that timed out (a workgroup never ran, e.g. on a device shared with a
 * kernel that holds compute units) or for value codebook entries outside the
 * supported range.  Unlike every other call this one synchronises: it waits
 * for `stream`, copies the word to *flags and, when `clear` is nonzero,
 * zeroes it.  Errors: LVQ_ERR_INVALID_ARG (null or misaligned workspace,
 * null flags), LVQ_ERR_HIP. */
lvq_status lvq_decode_status(void *workspace, uint32_t *flags, int32_t clear, void *stream);

/* Which (layer, sequence, query head) and which split role workgroup
 * `workgroup` of a decode launch of n_layers (1..16) layers takes, for
 * max_ctx_len with exact windows (host arithmetic: the mapping the kernel
 * computes from its dispatch index).  Roles 0 .. n-1 of a (layer, b, h) are
 * ordered by dispatch index; where the launch merges by window workgroups,
 * role n-1 merges, so it is the member of its group dispatched last.  With
 * one workgroup per (b, h) and 2 <= B <= 256 the kernel assigns sequences
 * by length at run time, and `seq` is then a position in that order.  Where
 * a workgroup serves two query heads (lvq_decode_heads_per_workgroup), `head`
 * is the first of them and the groups are (layer, b, head pair).
 * Returns the role, or -1 for an invalid config or workgroup index. */
int32_t lvq_decode_role(const lvq_config *cfg, int32_t n_layers, int32_t max_ctx_len,
                        int32_t workgroup, int32_t *layer, int32_t *seq, int32_t *head);

/* Number of workgroups per (b, h) that lvq_decode_attn launches for
 * max_ctx_len with exact windows (vq_len == NULL), per (b, head pair) when
 * lvq_decode_heads_per_workgroup is 2; host arithmetic only; 0 on an invalid
 * config. */
int32_t lvq_decode_splits(const lvq_config *cfg, int32_t max_ctx_len);

/* Query heads each decode workgroup serves (1 or 2, see
 * lvq_config.decode_heads_per_group) for a launch of n_layers layers
 * (1..LVQ_MAX_LAYERS) and max_ctx_len; host arithmetic only; 0 on an invalid
 * config or when decode_heads_per_group = 2 is not possible. */
int32_t lvq_decode_heads_per_workgroup(const lvq_config *cfg, int32_t n_layers, int32_t max_ctx_len);

/* How many of those workgroups take the bf16 window slots instead of a VQ
 * chunk (0: every workgroup takes a VQ chunk and a share of the window
 * slots); same arguments and conventions as lvq_decode_splits, -1 on an
 * invalid config. */
int32_t lvq_decode_window_groups(const lvq_config *cfg, int32_t max_ctx_len);

/* Static, NUL-terminated description of a status code. */
const char *lvq_status_string(lvq_status status);

#ifdef __cplusplus
}
#endif

#endif /* LOOPVQ_H */
