/*
 * na.h — C ABI of the MI355X (gfx950) N-dimensional local-attention library.
 *
 * Forward pass of softmax attention restricted to a local neighbourhood of each
 * query on a 1-D, 2-D or 3-D token grid ("pi-Attention: Online Efficient Sparse
 * Transformers for Long-Context Modeling", Section 3.2, Eqs. 4-5: the full sum
 * of Eq. 3 replaced by a sum over the neighbourhood), computed as block-sparse
 * fused attention: the token sequence is cut into query tiles and key/value
 * tiles, every (query tile, key/value tile) pair is classified once as empty,
 * partial or full ("Hilbert-Guided Sparse Local Attention", "Methodology in
 * Plain English"), empty pairs are skipped and only partial pairs are masked
 * element by element.
 *
 * Patterns covered (per pattern dimension: window, left offset, stride,
 * dilation, causal flag, border rule):
 *   - neighbourhood attention, window shifted inside at the borders, with
 *     strided and dilated forms ("Generalized Neighborhood Attention",
 *     abstract);
 *   - sliding-window / band attention cut at the borders, causal or not
 *     ("pi-Attention", Eq. 5);
 *   - sliding tile attention: tile order plus a strided window whose stride is
 *     the tile ("ENA: Efficient N-dimensional Attention", reading notes);
 *   - blocked (window) attention: stride = window, cut at the borders;
 *   - Hilbert-ordered window / slide / neighbourhood attention: tokens of a 2-D
 *     grid reordered along a Hilbert curve, pattern formed on the 1-D curve
 *     position ("Hilbert-Guided Sparse Local Attention", abstract).
 *
 * Conventions
 *   - Tensors q, k, v, out are [B, H, N, D] with D contiguous; na_tensor carries
 *     the base pointer and the element strides of the B, H and N axes.  Tokens
 *     are always in row-major grid order (last grid dimension fastest), also
 *     for Hilbert and tiled orders: reordering is internal.
 *   - lse is float32 [B, H, N], contiguous, row-major token order: the natural
 *     log of the sum over the neighbourhood of exp(scale * q.k).
 *   - All device pointers are caller-owned HIP device memory on the current
 *     device; `stream` is a hipStream_t (NULL = the null stream).  Work is
 *     enqueued asynchronously; nothing synchronises.
 *   - Every call returns an na_status; nothing throws across this boundary.
 *     Arguments are validated on the host before anything is enqueued; a
 *     failed validation touches no device memory.  na_last_error() gives a
 *     thread-local detail string for the last failure.
 */
#ifndef NA_H
#define NA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NA_ABI_VERSION 7

typedef enum {
    NA_OK = 0,
    NA_ERR_INVALID_ARG = 1,   /* malformed descriptor, pointer, size or stride */
    NA_ERR_UNSUPPORTED = 2,   /* valid, but no kernel variant for it (never a silent fallback) */
    NA_ERR_OUT_OF_MEMORY = 3, /* host or device allocation failed */
    NA_ERR_DEVICE = 4,        /* a HIP call or kernel launch failed; see na_last_error() */
    NA_ERR_PLAN_MISMATCH = 5  /* tensors or flags do not match the plan */
} na_status;

/* Token orders along which tiles are cut. */
enum {
    NA_ORDER_ROW_MAJOR = 0, /* row-major grid order */
    NA_ORDER_TILED = 1,     /* tile by tile (tile extents in na_plan_desc.tile), row-major inside */
    NA_ORDER_HILBERT = 2    /* 2-D grid along a Hilbert curve that starts at (row 0, col 0) and
                               ends at (row 0, cols-1); the pattern is 1-D over the curve position.
                               On power-of-two squares the classic curve; on any other rows x cols
                               grid its generalisation: blocks cut into the classic four-quadrant U
                               (or, when more than twice as long as wide, into two halves along the
                               travel direction) at even cut points where possible, so every step
                               is to a 4-neighbour unless cols is odd and rows even (then exactly
                               one step is diagonal) */
};

/* How pi-Attention's online partner combines with the local window
 * ("pi-Attention: Online Efficient Sparse Transformers for Long-Context
 * Modeling", Sections 3.4-3.5). */
enum {
    NA_SKIP_UNION = 0,        /* one softmax over the union of the window and the partners
                                 (Eqs. 8-11) */
    NA_SKIP_FIXED_FUSION = 1, /* one softmax over the union of z + log(alpha) on window keys and
                                 z + log(1 - alpha) on partners outside the window (Eqs. 16-17);
                                 lse is the log-sum-exp of those logits */
    NA_SKIP_SEPARATE = 2      /* a softmax over the window and one over the partners (Eq. 15);
                                 out is the sum of the two weighted averages, lse the window's */
};

/* Border rule of a pattern dimension. */
enum {
    NA_BOUND_CLAMP = 0,   /* the window is shifted to lie inside the axis (neighbourhood attention) */
    NA_BOUND_TRUNCATE = 1 /* the window is cut at the axis ends (band / slide attention) */
};

enum { NA_BF16 = 0, NA_F32 = 1 };

/* na_plan_create flags */
#define NA_PLAN_HOST_ONLY 1u /* build the tile map on the host only: no device upload; the plan can
                                be inspected but not run */

/* na_forward flags */
#define NA_FWD_PERMUTE_PASSES 1u /* for non-row-major orders: gather q, k, v into sequence order with
                                    the permute kernel, attend on contiguous tiles, scatter out and
                                    lse back (needs na_forward_workspace_bytes of workspace). Default:
                                    the attention kernel gathers and scatters rows itself. */
#define NA_FWD_SPLIT_TAIL 2u /* for the bf16 kernels without fixed fusion (and, at q_block 64,
                                128 or 256, without the separate softmax, whose partner branch
                                those kernels add in their epilogue): the r query tiles of the
                                last, partly filled round
                                of workgroups (r = tiles mod resident_workgroups of the plan's
                                stats) each run as s workgroups, each over one contiguous share of
                                the tile's key/value walk, writing unnormalised partial results
                                (fp32) that a second kernel merges.  s (2 to 16, r s at most four
                                rounds) minimises ceil(r s / resident) / s, the length of the
                                shares' rounds in whole-tile rounds; no split unless that is at
                                most 1/2 (each share pays its own Q load and pipeline fill).
                                Smaller problems (fewer tiles than one round) split every tile.
                                Needs na_forward_workspace_bytes of workspace (four rounds of
                                shares, independent of B and H); no effect on other launches. */

/*
 * Plan descriptor.  Pattern dimensions are the grid dimensions, except for
 * NA_ORDER_HILBERT where there is one pattern dimension: the curve position,
 * of length N.  For pattern dimension d with length L, a query at coordinate x
 * attends the keys y with
 *     c   = ((x' + shift) / stride) * stride - shift + stride / 2   (x' = x / dilation;
 *                                        the group's last position, + stride - 1, when causal)
 *     lo  = c - left, hi = lo + window                 (left = window_left, or window / 2,
 *                                                       or window - 1 when causal)
 *     clamp:    [lo, hi) shifted to lie inside [0, L'), or all of [0, L') if window >= L'
 *     truncate: [lo, hi) cut to [0, L')
 * evaluated on the sub-grid of positions congruent to x modulo dilation (L' its length), and
 * the N-D set is the Cartesian product of the per-dimension sets.  A causal dimension uses
 * left = window - 1 and truncation, and its stride groups are led by their last position, so a
 * group of `stride` positions (a chunk of frames, say) attends to itself and the window - stride
 * positions before it (block-causal); with stride 1 this is plain causal attention.
 */
typedef struct {
    int32_t ndim;           /* grid dimensions, 1..3 */
    int32_t grid[3];        /* grid extents, slowest first; N = product, N < 2^31 */
    int32_t order;          /* NA_ORDER_* */
    int32_t tile[3];        /* NA_ORDER_TILED: tile extents (>= 1) */
    int32_t window[3];      /* window length per pattern dimension (>= 1) */
    int32_t window_left[3]; /* window start offset; -1 = window / 2 (window - 1 if causal) */
    int32_t stride[3];      /* >= 1; 1 = plain sliding window */
    int32_t dilation[3];    /* >= 1 */
    int32_t causal[3];      /* 0 / 1 */
    int32_t boundary[3];    /* NA_BOUND_* (ignored for causal dimensions) */
    int32_t q_block;        /* query tile length in tokens, 0 = library default (fp32: 32;
                               bf16: 256 at head_dim 128, else 128) */
    int32_t kv_block;       /* key/value tile length in tokens, 0 = library default */
    int32_t head_dim;       /* D */
    int32_t dtype;          /* NA_BF16 or NA_F32 */
    int32_t shift[3];       /* phase of the stride groups, 0 <= shift < stride: groups are
                               [k*stride - shift, (k+1)*stride - shift).  With stride = window and
                               truncation, shift = window / 2 gives shifted (Swin-style) windows,
                               the shifted-window form of the Hilbert page's window attention */
    int32_t skip;           /* pi-Attention's online long-range partner (Eqs. 8-9): a query at
                               pattern position x also attends x - skip (0 = no partner); only for
                               one pattern dimension (1-D grids, Hilbert order), else
                               NA_ERR_UNSUPPORTED; partners outside the sequence do not exist */
    int32_t skip_both;      /* 1: also x + skip (bidirectional) */
    int32_t skip_mode;      /* NA_SKIP_* */
    float skip_prior;       /* alpha of NA_SKIP_FIXED_FUSION, 0 < alpha < 1 */
} na_plan_desc;

typedef struct {
    int64_t n_tokens;
    int64_t q_block, kv_block;
    int64_t n_q_tiles, n_kv_tiles;
    int64_t n_empty, n_partial, n_full; /* over all n_q_tiles * n_kv_tiles pairs */
    int64_t attended_pairs;             /* sum over queries of |neighbourhood|, per (batch, head);
                                           with a skip partner |window u partners|, or
                                           |window| + |partners| for NA_SKIP_SEPARATE */
    int64_t resident_workgroups;        /* workgroups of the plan's forward kernel resident on its
                                           device at once (compute units x workgroups per unit),
                                           the round NA_FWD_SPLIT_TAIL balances; 0 for host-only
                                           plans and kernels without that mode */
} na_plan_stats;

/* Speedup bounds of a pattern over dense attention of the same length and
 * tiles, from the tile map alone. */
typedef struct {
    double flop;            /* N^2 / attended pairs: what counting flops promises */
    double tile;            /* (n_q_tiles * n_kv_tiles) / non-empty tile pairs: what a kernel that
                               skips empty tiles and pays in full for every other one can reach */
    double useful_fraction; /* attended pairs / token pairs inside the non-empty tiles (ragged
                               last tiles at their true size); 1 for a perfectly block-sparse map */
} na_plan_bounds;

typedef struct {
    void* ptr;                          /* device pointer to element [0, 0, 0, 0] */
    int64_t stride_b, stride_h, stride_n; /* in elements; the D axis has stride 1 */
} na_tensor;

typedef struct na_plan_s* na_plan_t;

/* Build a plan: validate the descriptor, build the token order, classify every
 * (query tile, key/value tile) pair by interval arithmetic (exact: ambiguous
 * pairs are counted element by element), store the non-empty pairs per query
 * tile in CSR form, and (unless NA_PLAN_HOST_ONLY) upload order, CSR and the
 * per-token mask tables to the current device.  The plan owns all of it and is
 * immutable afterwards; it may be used from several streams at once.
 * Defined by: the block classes empty / partial / full and the reordering
 * path computed once and cached ("Hilbert-Guided Sparse Local Attention",
 * Methodology in Plain English); tiles sharing one window with the tile equal
 * to the kernel block ("ENA: Efficient N-dimensional Attention", core claim).
 * desc and plan are caller-owned host memory; *plan receives a handle the
 * caller releases with na_plan_destroy.
 * Returns NA_ERR_INVALID_ARG for a malformed descriptor, NA_ERR_UNSUPPORTED for
 * a Hilbert order on a grid that is not 2-D, NA_ERR_OUT_OF_MEMORY or
 * NA_ERR_DEVICE if a host or device allocation or upload fails (nothing is
 * leaked).  With the environment variable NA_LOG=1 (read once per process)
 * each created plan's statistics and build time go to stderr as one line;
 * NA_LOG=2 adds one line per na_forward launch (grid, whole tiles, split
 * shares).  Otherwise the library prints nothing. */
na_status na_plan_create(const na_plan_desc* desc, uint32_t flags, na_plan_t* plan);

/* Release a plan (host and device memory).  The caller must first make sure
 * that no enqueued work still uses it.  NULL is accepted. */
na_status na_plan_destroy(na_plan_t plan);

/* Tile-map statistics into caller-owned host memory (same source as
 * na_plan_create); attended_pairs sets the effective flops 4 * D * pairs * B * H. */
na_status na_plan_get_stats(na_plan_t plan, na_plan_stats* stats);

/* Speedup bounds of the plan's tile map (the realistic-bound simulator that
 * "Generalized Neighborhood Attention", Abstract, describes), into
 * caller-owned host memory.  NA_ERR_INVALID_ARG on NULL arguments. */
na_status na_plan_get_bounds(na_plan_t plan, na_plan_bounds* bounds);

/* Dense class matrix uint8 [n_q_tiles][n_kv_tiles]: 0 empty, 1 partial, 2 full
 * ("Hilbert-Guided Sparse Local Attention", Methodology in Plain English: a
 * block is empty, full, or partial and needs element masks), into
 * caller-owned host memory; n must be at least n_q_tiles * n_kv_tiles
 * (NA_ERR_INVALID_ARG otherwise). */
na_status na_plan_get_classes(na_plan_t plan, uint8_t* host_classes, size_t n);

/* perm[p] = row-major token at sequence position p (the order tokens are
 * reordered into, e.g. along the Hilbert curve: "Hilbert-Guided Sparse Local
 * Attention", Abstract), into caller-owned host memory; n must be >= N
 * (NA_ERR_INVALID_ARG otherwise). */
na_status na_plan_get_order(na_plan_t plan, int32_t* host_perm, size_t n);

/* Workspace bytes na_forward needs for (B, H) with the given flags (0 for the
 * default fused path): the permute passes' gathered q, k, v, out and lse,
 * then the split tail's shares (4 x resident workgroups x q_block x
 * (head_dim + 2) fp32 values), each part rounded up to 256 bytes. */
size_t na_forward_workspace_bytes(na_plan_t plan, int64_t B, int64_t H, uint32_t flags);

/* out = softmax attention of q over its neighbourhood keys/values, lse as
 * above: out_i = sum_j exp(z_ij - lse_i) v_j over the neighbourhood of i, with
 * z_ij = scale q_i . k_j ("pi-Attention", Section 3.1, Eqs. 1-3, restricted
 * to the neighbourhood as in Section 3.2, Eqs. 4-5).  q, k, v, out are
 * caller-owned device tensors and lse a caller-owned device buffer; nothing is
 * allocated (the permute passes and the split tail use the caller's
 * workspace, >= na_forward_workspace_bytes, 256-byte aligned).  Flags: 0,
 * NA_FWD_PERMUTE_PASSES, NA_FWD_SPLIT_TAIL or both.  q, k, v, out share the
 * plan's dtype and head_dim; lse may be NULL;
 * scale must be finite and positive (NA_ERR_INVALID_ARG otherwise).
 * Returns NA_ERR_PLAN_MISMATCH if the plan was built host-only, and
 * NA_ERR_UNSUPPORTED if no kernel matches (dtype, head_dim, q_block,
 * kv_block): bf16 with head_dim 64 or 128 and (q_block, kv_block) =
 * (128, 64), (192, 64) or (256, 64), (64, 64) at head_dim 64 and (384, 64) at head_dim 128;
 * fp32 with head_dim 32 or 64 and (32, 32).  Fixed fusion (NA_SKIP_FIXED_FUSION) runs in bf16 only, at q_block 128
 * or 256 (or 64 at head_dim 64).  The separate-softmax mode adds each query's
 * partner softmax to out: in the attention kernel's epilogue for bf16 at every
 * q_block except 192, otherwise in a second kernel enqueued after it.
 * In bf16 the probabilities are rounded to bf16 for the P.V product only; the
 * row sum (and so lse) adds them in fp32.
 * Inputs must be finite.  The kernels are built without NaN semantics (maxima
 * and comparisons assume none), and a masked key still enters the P.V product
 * with probability 0, so a NaN or infinity anywhere in q, k or v leaves out and
 * lse unspecified (not a fault) for every query whose query tile visits the key
 * tile that holds it; other queries are unaffected. */
na_status na_forward(na_plan_t plan, int64_t B, int64_t H, const na_tensor* q,
                     const na_tensor* k, const na_tensor* v, const na_tensor* out, float* lse,
                     float scale, uint32_t flags, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Workspace bytes na_backward needs for (B, H): the row sums
 * delta_i = dout_i . out_i, fp32 [B][H][N] (256-byte multiple). */
size_t na_backward_workspace_bytes(na_plan_t plan, int64_t B, int64_t H);

/* Gradients of sum_i dout_i . out_i with respect to q, k and v, where out is
 * the attention of na_forward over the same plan.  The softmax Jacobian is
 * that of the "pi-Attention" page (gradient analysis of adaptive fusion,
 * Eq. 23) restricted to the neighbourhood:
 *     P_ij  = exp(scale q_i . k_j - lse_i),  dP_ij = dout_i . v_j,
 *     dS_ij = P_ij (dP_ij - delta_i),        delta_i = dout_i . out_i,
 *     dq_i  = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i,
 *     dv_j  = sum_i P_ij dout_i.
 * Inputs: q, k, v, out, dout (plan dtype and head_dim, layout rules of
 * na_forward) and lse, the fp32 [B][H][N] output of na_forward for the same
 * q, k, v and scale.  Outputs dq, dk, dv: every element is written (zero for
 * keys no query attends and for queries whose neighbourhood is empty); they
 * must not overlap the inputs.  workspace: >= na_backward_workspace_bytes,
 * 256-byte aligned, caller-owned; no allocation happens.  bf16 only, head_dim
 * 64 or 128, (q_block, kv_block) = (128, 64) or (256, 64); other plans return
 * NA_ERR_UNSUPPORTED.  With a skip partner: the union mode is an ordinary
 * neighbourhood; fixed fusion adds its constant log-priors to the recomputed
 * logits (the softmax Jacobian is unchanged); the separate-softmax mode
 * computes the window branch's gradients with that branch's own row sums and
 * adds the partner branch's (two more kernels; lse is the window branch's, as
 * na_forward returns it).  P and dS are rounded to bf16 before their MFMA
 * products, accumulation is fp32.  Asynchronous on stream. */
na_status na_backward(na_plan_t plan, int64_t B, int64_t H, const na_tensor* q,
                      const na_tensor* k, const na_tensor* v, const na_tensor* out,
                      const na_tensor* dout, const float* lse, const na_tensor* dq,
                      const na_tensor* dk, const na_tensor* dv, float scale, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Size of the fixed device scratch of na_backward_noalloc: 16 MiB per GPU,
 * the delta rows of B * H * N <= 4,194,304 queries. */
#define NA_BACKWARD_NOALLOC_MAX_BYTES (16u << 20)

/* na_backward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without the workspace, the same kernels and results.  Its
 * delta rows go to a fixed scratch array in the library's static device data,
 * one per GPU, held until the process ends; the entry point calls no
 * hipMalloc, hipFree or allocating library routine.  Every element of the
 * scratch is written before it is read, so nothing needs clearing between
 * calls.  Calls on one GPU share that GPU's scratch: two calls that overlap in
 * time on one GPU (different streams, or host threads without ordering) race
 * and give wrong gradients; order them on one stream.  Returns
 * NA_ERR_INVALID_ARG when na_backward_workspace_bytes(plan, B, H) exceeds
 * NA_BACKWARD_NOALLOC_MAX_BYTES (checked before any device call), NA_ERR_DEVICE
 * if the scratch address cannot be found, and otherwise what na_backward
 * returns for the same arguments. */
na_status na_backward_noalloc(na_plan_t plan, int64_t B, int64_t H, const na_tensor* q,
                              const na_tensor* k, const na_tensor* v, const na_tensor* out,
                              const na_tensor* dout, const float* lse, const na_tensor* dq,
                              const na_tensor* dk, const na_tensor* dv, float scale,
                              void* stream);

/* Row gather along the plan's order: out[b, h, p, :] = in[b, h, perm[p], :]
 * (inverse = 0) or out[b, h, perm[p], :] = in[b, h, p, :] (inverse = 1), for
 * the plan's dtype and head_dim: the reordering of tokens along the curve and
 * back ("Hilbert-Guided Sparse Local Attention", Abstract and Methodology in
 * Plain English).  in and out are caller-owned device tensors and must not
 * overlap.  NA_ERR_UNSUPPORTED for a plan whose order is the identity,
 * NA_ERR_PLAN_MISMATCH for a host-only plan or another device, NA_ERR_DEVICE if
 * the launch fails.  Asynchronous on stream. */
na_status na_permute(na_plan_t plan, int64_t B, int64_t H, const na_tensor* in,
                     const na_tensor* out, int32_t inverse, void* stream);

/* Static name of a status code ("unknown status" for other values). */
const char* na_status_string(na_status status);
/* Detail of the calling thread's last failure (valid until its next call). */
const char* na_last_error(void);
/* NA_ABI_VERSION the library was built with; a binding compares it with the
 * header it mirrors. */
int32_t na_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
