/*
 * Plain fp64 CPU oracle for N-dimensional local attention: the forward pass
 * and its gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this code; it exists so that tests, the smoke check and the CPU
 * baseline of the benchmark have an independent, obviously correct
 * implementation to compare against.  It shares no source with the GPU
 * library: its descriptor types, its neighbourhood rules, its Hilbert curve
 * and its tile classification are all written separately from their
 * definitions.
 *
 * Everything is evaluated by explicit enumeration: for every query token the
 * set of attended keys is listed one by one from the per-dimension rules,
 * then softmax attention is evaluated over that list in double precision.
 */
#ifndef NA_ORACLE_H
#define NA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kind of a per-dimension neighbourhood rule. */
enum {
    ORC_WINDOW  = 0, /* sliding window of w positions starting at x - left,
                        shifted inside the axis (clamp) or cut at the ends
                        (truncate); optional stride leader and dilation */
    ORC_BLOCKED = 1, /* non-overlapping windows of w positions */
    ORC_STA     = 2  /* sliding tile: tiles of `tile` positions, the query's
                        tile attends `wt` whole tiles, shifted inside */
};

/* Token order along which the sequence (and therefore the tiles) run. */
enum {
    ORC_ORDER_ROW_MAJOR = 0,
    ORC_ORDER_TILED     = 1, /* tile by tile, row-major inside a tile */
    ORC_ORDER_HILBERT   = 2  /* 2-D grid, generalised Hilbert curve (orc_hilbert_grid) */
};

typedef struct {
    int32_t kind;
    int32_t clamp;    /* ORC_WINDOW: 1 = shift inside, 0 = truncate */
    int64_t w;        /* window length in positions (ORC_WINDOW, ORC_BLOCKED) */
    int64_t left;     /* ORC_WINDOW: window starts at x - left */
    int64_t stride;   /* ORC_WINDOW: group size sharing one window (1 = none) */
    int64_t dil;      /* ORC_WINDOW: dilation (1 = none) */
    int64_t tile;     /* ORC_STA: tile length */
    int64_t wt;       /* ORC_STA: window length in tiles */
    int64_t shift;    /* ORC_WINDOW groups / ORC_BLOCKED windows start at positions
                         congruent to -shift (0 <= shift < stride or w) */
    int64_t causal;   /* ORC_WINDOW: 1 = the window ends at the group's last position
                         (set with left = w - 1 and clamp = 0) */
} orc_rule;

typedef struct {
    int32_t ndim;        /* grid dimensions, 1..3 */
    int64_t grid[3];     /* extents, slowest first; N = product */
    int32_t order;       /* ORC_ORDER_* */
    int64_t tile[3];     /* ORC_ORDER_TILED: tile extents */
    /* Rules: for ROW_MAJOR / TILED orders one rule per grid dimension, applied
       to grid coordinates.  For HILBERT order a single rule (rule[0]) applied
       to the 1-D position along the curve, with axis length N. */
    orc_rule rule[3];
    /* pi-Attention's online long-range partner ("pi-Attention", Section 3.4,
       Eqs. 8-9; 1-D patterns only: 1-D grids or HILBERT order): query position
       x also attends x - skip (and x + skip when skip_both), when inside the
       sequence.  skip = 0: none.  skip_mode picks how the local set N_r and the
       partner set N_pi are combined (Section 3.5). */
    int64_t skip;
    int32_t skip_both;
    int32_t skip_mode;   /* ORC_SKIP_* */
    double skip_prior;   /* alpha of ORC_SKIP_FIXED_FUSION, in (0, 1) */
} orc_spec;

enum {
    ORC_SKIP_UNION = 0,        /* one softmax over U = N_r u N_pi (Eqs. 10-11) */
    ORC_SKIP_FIXED_FUSION = 1, /* one softmax over U of z + log(alpha) on N_r keys and
                                  z + log(1 - alpha) on the other keys (Eqs. 16-17) */
    ORC_SKIP_SEPARATE = 2      /* a softmax over N_r and one over N_pi (Eq. 15); the output
                                  is the sum of the two weighted averages (Eq. 11 with the
                                  weights of Eq. 15) and lse is the N_r branch's */
};

/* Number of tokens N. */
int64_t orc_num_tokens(const orc_spec* s);

/* perm[p] = row-major token index at sequence position p (length N). */
int orc_order(const orc_spec* s, int64_t* perm);

/* Hilbert curve over an n x n grid (n a power of two), built by recursive
   quadrant subdivision.  perm[p] = row*n + col of the p-th cell. */
int orc_hilbert(int64_t n, int64_t* perm);

/* Generalised Hilbert curve over a rows x cols grid (any sizes >= 1): the
   classic curve on power-of-two squares; otherwise the same quadrant U, or two
   halves along the travel direction for blocks more than twice as long as
   wide, split so that steps are 4-neighbour whenever the block's end corners
   allow it (one diagonal step otherwise).  Starts at (0, 0); ends at
   (0, cols - 1) when cols >= 2.  perm[p] = row*cols + col.  This is the order
   of HILBERT specs. */
int orc_hilbert_grid(int64_t rows, int64_t cols, int64_t* perm);

/* Neighbourhood of the 1-D rule at coordinate x on an axis of length len.
   Writes the ascending list of positions to out (capacity len) and returns
   its size. */
int64_t orc_rule_set(const orc_rule* r, int64_t len, int64_t x, int64_t* out);

/* The online partners N_pi(i) of row-major token i, ascending row-major
   token indices; returns their number (0 without skip). */
int64_t orc_partners(const orc_spec* s, const int64_t* perm, const int64_t* pos_of_token,
                     int64_t i, int64_t* out);

/* Neighbourhood N(i) of row-major token i, as ascending row-major token
   indices.  out must hold N entries.  pos_of_token / perm may be NULL unless
   the order is HILBERT (they are the inverse pair from orc_order).  With a
   skip partner this is the union U(i) (Eq. 8), except for the separate-softmax
   variant, where it is the local set N_r(i) alone. */
int64_t orc_neighbors(const orc_spec* s, const int64_t* perm,
                      const int64_t* pos_of_token, int64_t i, int64_t* out);

/* Total attended (query, key) pairs per (batch, head) (for the separate-softmax
   variant: |N_r(i)| + |N_pi(i)| summed). */
int64_t orc_attended_pairs(const orc_spec* s);

/* Softmax attention restricted to N(i).
   q, k, v: contiguous [B][H][N][D]; dtype 0 = bf16 bit patterns (uint16),
   1 = float32, 2 = float64.  rows: the row-major query tokens to evaluate (nrows of them),
   or NULL with nrows = N for all.  out: [B][H][nrows][D] fp64,
   lse: [B][H][nrows] fp64 (natural log of the sum of exp of scaled logits).
   threads <= 0 uses the OpenMP default.  Returns 0 on success. */
int orc_attention(const orc_spec* s, int64_t B, int64_t H, int64_t D, int32_t dtype,
                  const void* q, const void* k, const void* v, double scale,
                  const int64_t* rows, int64_t nrows, double* out, double* lse,
                  int32_t threads);

/* Gradients of sum_i dout_i . out_i with respect to q, k, v, where out is the
   attention above over all N rows.  q, k, v, dout: contiguous [B][H][N][D] of
   one dtype (codes as above); dq, dk, dv: [B][H][N][D] fp64.  Rows with an
   empty neighbourhood contribute nothing.  Returns 0 on success. */
int orc_attention_backward(const orc_spec* s, int64_t B, int64_t H, int64_t D, int32_t dtype,
                           const void* q, const void* k, const void* v, const void* dout,
                           double scale, double* dq, double* dk, double* dv, int32_t threads);

/* dq of the same gradients for the listed row-major query tokens only:
   dq [B][H][nrows][D] fp64 (dq_i needs nothing beyond row i's neighbourhood). */
int orc_attention_backward_dq_rows(const orc_spec* s, int64_t B, int64_t H, int64_t D,
                                   int32_t dtype, const void* q, const void* k, const void* v,
                                   const void* dout, double scale, const int64_t* rows,
                                   int64_t nrows, double* dq, int32_t threads);

/* dk and dv of the same gradients for the listed row-major key tokens only
   (distinct, in [0, N)): dk, dv [B][H][nkeys][D] fp64.  Returns 0 on success,
   -2 for a key out of range or listed twice. */
int orc_attention_backward_kv_rows(const orc_spec* s, int64_t B, int64_t H, int64_t D,
                                   int32_t dtype, const void* q, const void* k, const void* v,
                                   const void* dout, double scale, const int64_t* keys,
                                   int64_t nkeys, double* dk, double* dv, int32_t threads);

/* Tile classes over the sequence order: cls[qt * nkt + kt] in {0 empty,
   1 partial, 2 full}; nqt = ceil(N/q_block), nkt = ceil(N/kv_block).
   *pairs receives the attended-pair count.  Returns 0 on success. */
int orc_tile_classes(const orc_spec* s, int64_t q_block, int64_t kv_block,
                     uint8_t* cls, int64_t* pairs, int32_t threads);

/* Worker threads the OpenMP runtime would use. */
int32_t orc_max_threads(void);

#ifdef __cplusplus
}
#endif
#endif
