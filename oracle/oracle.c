/*
 * Plain fp64 CPU oracle for N-dimensional local attention (forward and its gradients).
 *
 * TEST INFRASTRUCTURE ONLY: called from the tests, the smoke check and the
 * CPU-baseline leg of the benchmark, never from the product path.  It shares
 * no code with the GPU library.
 *
 * Sources of each rule (pages as titled):
 *  - softmax attention over a key set, and the causal / bidirectional local
 *    neighbourhoods: "pi-Attention: Online Efficient Sparse Transformers for
 *    Long-Context Modeling", Section 3.1 (Eqs. 1-3) and Section 3.2 (Eqs. 4-5);
 *    invalid positions are excluded before the softmax (Appendix A, text after
 *    Eq. 34).
 *  - sliding tile attention (tiles share one window that moves tile by tile,
 *    shifted inside the grid): "ENA: Efficient N-dimensional Attention",
 *    reading notes ("What carries the argument", "Core claim").
 *  - neighbourhood attention with the window shifted inside at the borders,
 *    strided (grouped) and blocked windows: "Generalized Neighborhood
 *    Attention", abstract.  The stride leader and the dilation sub-grid rule are
 *    readings (the pages give only the names): a group of `stride` consecutive
 *    positions shares the window of its middle position; dilation runs the
 *    rule on the interleaved sub-grid of positions congruent to x.
 *  - pi-Attention's online long-range partner (pi-Attention, Section 3.4,
 *    Eqs. 8-11) and its fusion variants (Section 3.5: separate softmax,
 *    Eq. 15; fixed fusion, Eqs. 16-17).  The output of the separate variant
 *    is a reading: the page defines the two branch softmaxes only, and the
 *    output is taken as Eq. 11 with those weights (the two weighted averages
 *    added).
 *  - Hilbert reordering with windows / slides formed on the reordered 1-D
 *    sequence, and the empty / partial / full tile classes:
 *    "Hilbert-Guided Sparse Local Attention", "Methodology in Plain English"
 *    and "Key Contributions".
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }
static int64_t imax(int64_t a, int64_t b) { return a > b ? a : b; }
static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int32_t orc_max_threads(void) {
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}

int64_t orc_num_tokens(const orc_spec* s) {
    int64_t n = 1;
    for (int d = 0; d < s->ndim; ++d) n *= s->grid[d];
    return n;
}

/* Grid extent of dimension d, 1 beyond ndim. */
static int64_t extent(const orc_spec* s, int d) { return d < s->ndim ? s->grid[d] : 1; }

/* ------------------------------------------------------------------------ */
/* One-dimensional neighbourhood rules.                                     */
/* ------------------------------------------------------------------------ */

/* Sliding window on an axis of length L at coordinate x (Eq. 5 of the
   pi-Attention page generalised to a window of w positions that starts at
   x - left).  With clamp the window is shifted to lie inside the axis (the
   neighbourhood-attention border rule); without it the window is cut at the
   axis ends (positions outside are invalid and dropped).  Stride: positions are
   grouped `stride` at a time (groups start at positions congruent to -shift)
   and each group uses the window of its middle position (of its last position
   for a causal rule, whose window ends there).  Dilation: only positions congruent to x modulo `dil` take part,
   and the rule runs in the coordinates of that sub-grid. */
static int64_t window_set(const orc_rule* r, int64_t L, int64_t x, int64_t* out) {
    const int64_t dil = r->dil > 0 ? r->dil : 1;
    const int64_t stride = r->stride > 0 ? r->stride : 1;
    const int64_t g = x % dil;                 /* which interleaved sub-grid */
    const int64_t xl = x / dil;                /* coordinate inside it */
    const int64_t Lg = ceil_div(L - g, dil);   /* its length */
    /* group leader; with stride 1 every position leads its own group */
    const int64_t first = ((xl + r->shift) / stride) * stride - r->shift; /* group start */
    /* the middle position leads its group; a causal group is led by its last
       position, so every member sees the whole group */
    const int64_t centre = first + (r->causal ? stride - 1 : stride / 2);
    int64_t lo, hi;
    if (r->clamp) {
        if (r->w >= Lg) {
            lo = 0;
            hi = Lg;
        } else {
            lo = imin(imax(centre - r->left, 0), Lg - r->w);
            hi = lo + r->w;
        }
    } else {
        lo = imax(centre - r->left, 0);
        hi = imin(centre - r->left + r->w, Lg);
    }
    int64_t n = 0;
    for (int64_t t = lo; t < hi; ++t) out[n++] = g + dil * t;
    return n;
}

/* Non-overlapping windows of w positions; the first and last may be shorter.
   Window k covers [k*w - shift, (k+1)*w - shift): shift = 0 is plain window
   attention, shift > 0 the shifted windows that let neighbouring windows
   exchange information ("Hilbert-Guided Sparse Local Attention", Key
   Contributions: windows shifted along the 1-D sequence). */
static int64_t blocked_set(const orc_rule* r, int64_t L, int64_t x, int64_t* out) {
    const int64_t lo = imax(((x + r->shift) / r->w) * r->w - r->shift, 0);
    const int64_t hi = imin(((x + r->shift) / r->w + 1) * r->w - r->shift, L);
    int64_t n = 0;
    for (int64_t t = lo; t < hi; ++t) out[n++] = t;
    return n;
}

/* Sliding tile attention on one axis: the axis is cut into tiles of `tile`
   positions; the query's tile attends `wt` consecutive whole tiles centred on
   it, shifted so that the window stays inside the axis. */
static int64_t sta_set(const orc_rule* r, int64_t L, int64_t x, int64_t* out) {
    const int64_t T = ceil_div(L, r->tile);
    const int64_t t = x / r->tile;
    int64_t first, last; /* tile range [first, last) */
    if (r->wt >= T) {
        first = 0;
        last = T;
    } else {
        first = imin(imax(t - r->wt / 2, 0), T - r->wt);
        last = first + r->wt;
    }
    int64_t n = 0;
    for (int64_t p = first * r->tile; p < imin(last * r->tile, L); ++p) out[n++] = p;
    return n;
}

int64_t orc_rule_set(const orc_rule* r, int64_t len, int64_t x, int64_t* out) {
    switch (r->kind) {
        case ORC_WINDOW: return window_set(r, len, x, out);
        case ORC_BLOCKED: return blocked_set(r, len, x, out);
        case ORC_STA: return sta_set(r, len, x, out);
        default: return -1;
    }
}

/* ------------------------------------------------------------------------ */
/* Token orders.                                                            */
/* ------------------------------------------------------------------------ */

/* Emit the cells of a size x size block from corner (r, c), travelling first
   along direction u and turning into the block along direction v.  The block
   is split into four quadrants visited in a U: the start quadrant (whose own
   curve is transposed so that it ends next to the second one), the quadrant
   one half-step along v, the one diagonal to the start, and the one one
   half-step along u (whose curve is reversed and transposed so that it ends at
   the block's end corner, (size-1) steps along u from the start). */
static void hilbert_rec(int64_t n, int64_t size, int64_t r, int64_t c, int64_t ur, int64_t uc,
                        int64_t vr, int64_t vc, int64_t* perm, int64_t* k) {
    if (size == 1) {
        perm[(*k)++] = r * n + c;
        return;
    }
    const int64_t h = size / 2;
    hilbert_rec(n, h, r, c, vr, vc, ur, uc, perm, k);
    hilbert_rec(n, h, r + h * vr, c + h * vc, ur, uc, vr, vc, perm, k);
    hilbert_rec(n, h, r + h * vr + h * ur, c + h * vc + h * uc, ur, uc, vr, vc, perm, k);
    hilbert_rec(n, h, r + (h - 1) * vr + (2 * h - 1) * ur, c + (h - 1) * vc + (2 * h - 1) * uc,
                -vr, -vc, -ur, -uc, perm, k);
}

int orc_hilbert(int64_t n, int64_t* perm) {
    if (n < 1 || (n & (n - 1)) != 0) return -1;
    int64_t k = 0;
    /* Start at (row 0, col 0), end at (row 0, col n-1): u points along the
       columns, v down the rows. */
    hilbert_rec(n, n, 0, 0, 0, 1, 1, 0, perm, &k);
    return 0;
}

/* Generalised Hilbert curve over any rows x cols grid.  The pages name no
   curve for grids that are not power-of-two squares; this construction is a
   reading (documented with the library): it is the classic curve above on
   power-of-two squares, and elsewhere splits a block into the same four
   quadrants visited in the same U, or into two halves along its travel
   direction when the block is more than twice as long as it is wide, with
   split points chosen so that every step moves to a 4-neighbour whenever a
   path with the block's two end corners allows it.

   walk() emits the w x h block of cells o + i*a + j*b (0 <= i < w, 0 <= j < h;
   a and b unit vectors in (row, col)), starting at o and, when w >= 2, ending
   at o + (w-1)*a. */
typedef struct {
    int64_t cols;
    int64_t* perm;
    int64_t k;
} walk_out;

static void walk_emit(walk_out* out, int64_t r, int64_t c) {
    out->perm[out->k++] = r * out->cols + c;
}

/* Even split near the middle of a length >= 4: 2 * floor((w + 2) / 4), kept in
   [2, w - 2]. */
static int64_t even_half(int64_t w) {
    int64_t h = 2 * ((w + 2) / 4);
    if (h < 2) h = 2;
    if (h > w - 2) h = w - 2;
    return h;
}

static void walk(walk_out* out, int64_t r, int64_t c, int64_t ar, int64_t ac, int64_t br,
                 int64_t bc, int64_t w, int64_t h) {
    if (h == 1) { /* a straight run along a */
        for (int64_t i = 0; i < w; ++i) walk_emit(out, r + i * ar, c + i * ac);
        return;
    }
    if (w == 1) { /* only for a one-column grid: straight down b */
        for (int64_t j = 0; j < h; ++j) walk_emit(out, r + j * br, c + j * bc);
        return;
    }
    if (h == 2 && w == 2) { /* the U of the classic curve */
        walk_emit(out, r, c);
        walk_emit(out, r + br, c + bc);
        walk_emit(out, r + ar + br, c + ac + bc);
        walk_emit(out, r + ar, c + ac);
        return;
    }
    if (h == 2 && w == 3) { /* no 4-neighbour path joins these corners: one diagonal step */
        walk_emit(out, r, c);
        walk_emit(out, r + br, c + bc);
        walk_emit(out, r + ar, c + ac);
        walk_emit(out, r + ar + br, c + ac + bc);
        walk_emit(out, r + 2 * ar + br, c + 2 * ac + bc);
        walk_emit(out, r + 2 * ar, c + 2 * ac);
        return;
    }
    if (h == 2 || w > 2 * h) { /* long block: two halves, both travelling along a */
        const int64_t w1 = even_half(w);
        walk(out, r, c, ar, ac, br, bc, w1, h);
        walk(out, r + w1 * ar, c + w1 * ac, ar, ac, br, bc, w - w1, h);
        return;
    }
    /* Four quadrants: near-left (travelling along b), far-left and far-right
       (along a), near-right (back along -b, ending at the block's end corner).
       Left widths and the near height are even where they can be, which keeps
       every quadrant's own corners joinable by 4-neighbour steps. */
    int64_t w1, h2;
    if (w <= 3) {
        w1 = w - 1;
        h2 = 1;
    } else {
        w1 = even_half(w);
        h2 = h / 2 < w / 2 ? h / 2 : w / 2;
        if (h2 < 1) h2 = 1;
    }
    int64_t h1 = h - h2;
    if (w > 3 && h1 % 2 == 1) {
        if (h2 >= 2) {
            h1 += 1;
        } else {
            h1 -= 1;
        }
    }
    h2 = h - h1;
    const int64_t w2 = w - w1;
    walk(out, r, c, br, bc, ar, ac, h1, w1);
    walk(out, r + h1 * br, c + h1 * bc, ar, ac, br, bc, w1, h2);
    walk(out, r + w1 * ar + h1 * br, c + w1 * ac + h1 * bc, ar, ac, br, bc, w2, h2);
    walk(out, r + (w - 1) * ar + (h1 - 1) * br, c + (w - 1) * ac + (h1 - 1) * bc, -br, -bc, -ar,
         -ac, h1, w2);
}

int orc_hilbert_grid(int64_t rows, int64_t cols, int64_t* perm) {
    if (rows < 1 || cols < 1) return -1;
    walk_out out = {cols, perm, 0};
    /* Start at (row 0, col 0), travel along the columns (a), turn down the rows
       (b): as the classic curve. */
    walk(&out, 0, 0, 0, 1, 1, 0, cols, rows);
    return out.k == rows * cols ? 0 : -1;
}

int orc_order(const orc_spec* s, int64_t* perm) {
    const int64_t N = orc_num_tokens(s);
    if (s->order == ORC_ORDER_ROW_MAJOR) {
        for (int64_t i = 0; i < N; ++i) perm[i] = i;
        return 0;
    }
    if (s->order == ORC_ORDER_HILBERT) {
        if (s->ndim != 2) return -1;
        return orc_hilbert_grid(s->grid[0], s->grid[1], perm);
    }
    if (s->order == ORC_ORDER_TILED) {
        const int64_t g0 = extent(s, 0), g1 = extent(s, 1), g2 = extent(s, 2);
        const int64_t t0 = s->ndim > 0 ? s->tile[0] : 1;
        const int64_t t1 = s->ndim > 1 ? s->tile[1] : 1;
        const int64_t t2 = s->ndim > 2 ? s->tile[2] : 1;
        if (t0 < 1 || t1 < 1 || t2 < 1) return -1;
        int64_t k = 0;
        for (int64_t a = 0; a < g0; a += t0)
            for (int64_t b = 0; b < g1; b += t1)
                for (int64_t c = 0; c < g2; c += t2)
                    for (int64_t x = a; x < imin(a + t0, g0); ++x)
                        for (int64_t y = b; y < imin(b + t1, g1); ++y)
                            for (int64_t z = c; z < imin(c + t2, g2); ++z)
                                perm[k++] = (x * g1 + y) * g2 + z;
        return 0;
    }
    return -1;
}

/* ------------------------------------------------------------------------ */
/* Neighbourhoods of tokens.                                                */
/* ------------------------------------------------------------------------ */

static int cmp_i64(const void* a, const void* b) {
    const int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x > y) - (x < y);
}

/* The local set N_r(i): the pattern's neighbourhood. */
static int64_t local_neighbors(const orc_spec* s, const int64_t* perm,
                               const int64_t* pos_of_token, int64_t i, int64_t* out) {
    const int64_t N = orc_num_tokens(s);
    if (s->order == ORC_ORDER_HILBERT) {
        /* The rule acts on positions along the curve; keys are mapped back to
           row-major tokens. */
        const int64_t p = pos_of_token[i];
        const int64_t n = orc_rule_set(&s->rule[0], N, p, out);
        for (int64_t t = 0; t < n; ++t) out[t] = perm[out[t]];
        qsort(out, (size_t)n, sizeof(int64_t), cmp_i64);
        return n;
    }
    /* N-D: the set is the Cartesian product of the per-dimension sets. */
    const int64_t g0 = extent(s, 0), g1 = extent(s, 1), g2 = extent(s, 2);
    const int64_t c0 = i / (g1 * g2), c1 = (i / g2) % g1, c2 = i % g2;
    int64_t* s0 = (int64_t*)malloc(sizeof(int64_t) * (size_t)(g0 + g1 + g2));
    int64_t* s1 = s0 + g0;
    int64_t* s2 = s1 + g1;
    const orc_rule whole = {ORC_WINDOW, 1, 1, 0, 1, 1, 1, 1};
    const int64_t n0 = orc_rule_set(&s->rule[0], g0, c0, s0);
    const int64_t n1 = orc_rule_set(s->ndim > 1 ? &s->rule[1] : &whole, g1, c1, s1);
    const int64_t n2 = orc_rule_set(s->ndim > 2 ? &s->rule[2] : &whole, g2, c2, s2);
    int64_t n = 0;
    for (int64_t a = 0; a < n0; ++a)
        for (int64_t b = 0; b < n1; ++b)
            for (int64_t c = 0; c < n2; ++c) out[n++] = (s0[a] * g1 + s1[b]) * g2 + s2[c];
    free(s0);
    return n;
}

/* Inverse of perm. */
static int64_t* invert(const int64_t* perm, int64_t N) {
    int64_t* inv = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    for (int64_t p = 0; p < N; ++p) inv[perm[p]] = p;
    return inv;
}

/* N_pi(i) (pi-Attention, Eq. 9): the key pi positions back along the 1-D
   pattern axis, and pi positions ahead when both directions are fetched; only
   positions inside the sequence exist. */
int64_t orc_partners(const orc_spec* s, const int64_t* perm, const int64_t* pos_of_token,
                     int64_t i, int64_t* out) {
    if (s->skip <= 0) return 0;
    const int64_t N = orc_num_tokens(s);
    const int hil = s->order == ORC_ORDER_HILBERT;
    const int64_t x = hil ? pos_of_token[i] : i; /* 1-D: the token is the coordinate */
    int64_t n = 0;
    if (x - s->skip >= 0) out[n++] = x - s->skip;
    if (s->skip_both && x + s->skip < N) out[n++] = x + s->skip;
    for (int64_t a = 0; a < n; ++a)
        if (hil) out[a] = perm[out[a]];
    qsort(out, (size_t)n, sizeof(int64_t), cmp_i64);
    return n;
}

/* Is token j in the ascending list set[0..n)? */
static int contains(const int64_t* set, int64_t n, int64_t j) {
    int64_t lo = 0, hi = n;
    while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (set[mid] < j) lo = mid + 1; else hi = mid;
    }
    return lo < n && set[lo] == j;
}

int64_t orc_neighbors(const orc_spec* s, const int64_t* perm, const int64_t* pos_of_token,
                      int64_t i, int64_t* out) {
    int64_t n = local_neighbors(s, perm, pos_of_token, i, out);
    if (s->skip <= 0 || s->skip_mode == ORC_SKIP_SEPARATE) return n;
    /* U(i) = N_r(i) u N_pi(i) (Eq. 8): add the partners not already local */
    int64_t part[2];
    const int64_t np = orc_partners(s, perm, pos_of_token, i, part);
    const int64_t nl = n;
    for (int64_t a = 0; a < np; ++a)
        if (!contains(out, nl, part[a])) out[n++] = part[a];
    if (n > nl) qsort(out, (size_t)n, sizeof(int64_t), cmp_i64);
    return n;
}

/* The key sets over which query i takes a softmax, with an additive log-prior
   per key (pi-Attention, Section 3.5): branch 0 is U(i) (or N_r(i) for the
   separate variant), branch 1 exists only for the separate variant and is
   N_pi(i).  Returns the number of keys, or -1 if the branch does not exist.
   lp may be NULL when the caller needs no priors. */
static int64_t branch_keys(const orc_spec* s, const int64_t* perm, const int64_t* pos, int64_t i,
                           int branch, int64_t* nb, double* lp) {
    const int separate = s->skip > 0 && s->skip_mode == ORC_SKIP_SEPARATE;
    if (branch == 1 && !separate) return -1;
    const int64_t n = branch == 0 ? orc_neighbors(s, perm, pos, i, nb)
                                  : orc_partners(s, perm, pos, i, nb);
    if (lp) {
        for (int64_t a = 0; a < n; ++a) lp[a] = 0.0;
        if (s->skip > 0 && s->skip_mode == ORC_SKIP_FIXED_FUSION && n > 0) {
            /* delta_ij = z_ij + log(omega_ij), omega = alpha on N_r, 1 - alpha on
               the partners (Eq. 16) */
            int64_t* loc = (int64_t*)malloc(sizeof(int64_t) * (size_t)orc_num_tokens(s));
            const int64_t nl = local_neighbors(s, perm, pos, i, loc);
            for (int64_t a = 0; a < n; ++a)
                lp[a] = contains(loc, nl, nb[a]) ? log(s->skip_prior) : log(1.0 - s->skip_prior);
            free(loc);
        }
    }
    return n;
}

int64_t orc_attended_pairs(const orc_spec* s) {
    const int64_t N = orc_num_tokens(s);
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    if (orc_order(s, perm) != 0) {
        free(perm);
        return -1;
    }
    int64_t* pos = invert(perm, N);
    int64_t total = 0;
#pragma omp parallel reduction(+ : total)
    {
        int64_t* buf = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
#pragma omp for schedule(dynamic, 64)
        for (int64_t i = 0; i < N; ++i) {
            total += orc_neighbors(s, perm, pos, i, buf);
            if (s->skip > 0 && s->skip_mode == ORC_SKIP_SEPARATE)
                total += orc_partners(s, perm, pos, i, buf);
        }
        free(buf);
    }
    free(pos);
    free(perm);
    return total;
}

/* ------------------------------------------------------------------------ */
/* Attention (Eqs. 2-4 of the pi-Attention page over the set N(i)).          */
/* ------------------------------------------------------------------------ */

static double load_elem(const void* base, int32_t dtype, int64_t idx) {
    if (dtype == 2) return ((const double*)base)[idx];
    if (dtype == 1) return (double)((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int orc_attention(const orc_spec* s, int64_t B, int64_t H, int64_t D, int32_t dtype,
                  const void* q, const void* k, const void* v, double scale,
                  const int64_t* rows, int64_t nrows, double* out, double* lse,
                  int32_t threads) {
    const int64_t N = orc_num_tokens(s);
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    if (orc_order(s, perm) != 0) {
        free(perm);
        return -1;
    }
    int64_t* pos = invert(perm, N);
    const int64_t total = B * H * nrows;
    int err = 0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        int64_t* nb = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
        double* z = (double*)malloc(sizeof(double) * (size_t)N);
        double* qi = (double*)malloc(sizeof(double) * (size_t)D);
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        double* lp = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < total; ++t) {
            const int64_t bh = t / nrows, r = t % nrows;
            const int64_t i = rows ? rows[r] : r;
            if (i < 0 || i >= N) {
                err = 1;
                continue;
            }
            const int64_t head = bh * N * D;
            for (int64_t d = 0; d < D; ++d) qi[d] = load_elem(q, dtype, head + i * D + d);
            double* o = out + t * D;
            for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
            lse[t] = -INFINITY;
            /* One softmax per branch (one branch unless the separate-softmax
               variant); the output sums the branches' weighted averages. */
            for (int branch = 0; branch < 2; ++branch) {
                const int64_t n = branch_keys(s, perm, pos, i, branch, nb, lp);
                if (n <= 0) continue; /* no such branch, or an empty set: adds nothing */
                /* delta_ij = scale * q_i . k_j + log-prior  (Eq. 4, and Eq. 16 for
                   fixed fusion) */
                double m = -INFINITY;
                for (int64_t a = 0; a < n; ++a) {
                    const int64_t kj = head + nb[a] * D;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += qi[d] * load_elem(k, dtype, kj + d);
                    z[a] = scale * dot + lp[a];
                    if (z[a] > m) m = z[a];
                }
                /* alpha_ij = exp(delta_ij) / sum_j' exp(delta_ij') (Eq. 2, Eq. 10,
                   Eq. 17), written with the row maximum factored out; output =
                   sum_j alpha_ij v_j (Eq. 3, Eq. 11). */
                double l = 0.0;
                for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
                for (int64_t a = 0; a < n; ++a) {
                    const double e = exp(z[a] - m);
                    l += e;
                    const int64_t vj = head + nb[a] * D;
                    for (int64_t d = 0; d < D; ++d) acc[d] += e * load_elem(v, dtype, vj + d);
                }
                for (int64_t d = 0; d < D; ++d) o[d] += acc[d] / l;
                if (branch == 0) lse[t] = m + log(l);
            }
        }
        free(lp);
        free(acc);
        free(qi);
        free(z);
        free(nb);
    }
    free(pos);
    free(perm);
    return err ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Gradients of the restricted attention.                                   */
/* ------------------------------------------------------------------------ */

/* Gradient contributions of query i (row-major token) of one (batch, head)
   slice starting at element `head`, in the order of the definition:
     z_ij = scale q_i . k_j                       (pi-Attention, Eq. 4)
     P_ij = exp(z_ij) / sum_j' exp(z_ij')         (Eq. 2, over N(i))
     dP_ij = dout_i . v_j                         (Eq. 3 is linear in P)
     dz_ij = P_ij (dP_ij - sum_j' P_ij' dP_ij')   (softmax Jacobian, Eq. 23)
     dq_i += scale dz_ij k_j,  dk_j += scale dz_ij q_i,  dv_j += P_ij dout_i.
   dqi receives dq_i (D values, added to) and may be NULL.  dk / dv (the
   slice's rows, added to) may be NULL; with slot == NULL key j's row is row j,
   else it is row slot[j] and keys with slot[j] < 0 are not accumulated.
   nb, p, dp: scratch of N entries; qi, gi: scratch of D entries. */
static void grad_branch(const orc_spec* s, const int64_t* perm, const int64_t* pos, int64_t D,
                        int32_t dtype, const void* q, const void* k, const void* v,
                        const void* dout, double scale, int64_t head, int64_t i, int branch,
                        double* dqi, double* dk, double* dv, const int64_t* slot, int64_t* nb,
                        double* p, double* dp, double* qi, double* gi) {
    /* the log-priors of fixed fusion are constants: they change P, not the
       Jacobian of the softmax with respect to z.  dp holds them until the dP
       values overwrite it. */
    const int64_t n = branch_keys(s, perm, pos, i, branch, nb, dp);
    if (n <= 0) return; /* out_i = 0 (or no such branch) does not depend on q, k, v */
    for (int64_t d = 0; d < D; ++d) {
        qi[d] = load_elem(q, dtype, head + i * D + d);
        gi[d] = load_elem(dout, dtype, head + i * D + d);
    }
    double m = -INFINITY;
    for (int64_t a = 0; a < n; ++a) {
        const int64_t kj = head + nb[a] * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += qi[d] * load_elem(k, dtype, kj + d);
        p[a] = scale * dot + dp[a];
        if (p[a] > m) m = p[a];
    }
    double l = 0.0;
    for (int64_t a = 0; a < n; ++a) {
        p[a] = exp(p[a] - m);
        l += p[a];
    }
    double delta = 0.0;
    for (int64_t a = 0; a < n; ++a) {
        p[a] /= l;
        const int64_t vj = head + nb[a] * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += gi[d] * load_elem(v, dtype, vj + d);
        dp[a] = dot;
        delta += p[a] * dot;
    }
    for (int64_t a = 0; a < n; ++a) {
        const double dz = p[a] * (dp[a] - delta);
        const int64_t j = head + nb[a] * D;
        if (dqi)
            for (int64_t d = 0; d < D; ++d) dqi[d] += scale * dz * load_elem(k, dtype, j + d);
        const int64_t row = slot ? slot[nb[a]] : nb[a];
        if (row < 0) continue;
        for (int64_t d = 0; d < D; ++d) {
            if (dk) dk[row * D + d] += scale * dz * qi[d];
            if (dv) dv[row * D + d] += p[a] * gi[d];
        }
    }
}

/* All branches of query i (the separate-softmax variant has two independent
   softmaxes whose outputs add, so their gradients add). */
static void grad_row(const orc_spec* s, const int64_t* perm, const int64_t* pos, int64_t D,
                     int32_t dtype, const void* q, const void* k, const void* v,
                     const void* dout, double scale, int64_t head, int64_t i, double* dqi,
                     double* dk, double* dv, const int64_t* slot, int64_t* nb, double* p,
                     double* dp, double* qi, double* gi) {
    for (int branch = 0; branch < 2; ++branch)
        grad_branch(s, perm, pos, D, dtype, q, k, v, dout, scale, head, i, branch, dqi, dk, dv,
                    slot, nb, p, dp, qi, gi);
}

/* Every (batch, head) slice is owned by one thread, so the scatter into dk and
   dv needs no synchronisation. */
int orc_attention_backward(const orc_spec* s, int64_t B, int64_t H, int64_t D, int32_t dtype,
                           const void* q, const void* k, const void* v, const void* dout,
                           double scale, double* dq, double* dk, double* dv, int32_t threads) {
    const int64_t N = orc_num_tokens(s);
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    if (orc_order(s, perm) != 0) {
        free(perm);
        return -1;
    }
    int64_t* pos = invert(perm, N);
    const int64_t total = B * H * N * D;
    for (int64_t t = 0; t < total; ++t) dq[t] = dk[t] = dv[t] = 0.0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        int64_t* nb = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
        double* p = (double*)malloc(sizeof(double) * (size_t)N);
        double* dp = (double*)malloc(sizeof(double) * (size_t)N);
        double* qi = (double*)malloc(sizeof(double) * (size_t)D);
        double* gi = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t bh = 0; bh < B * H; ++bh) {
            const int64_t head = bh * N * D;
            for (int64_t i = 0; i < N; ++i)
                grad_row(s, perm, pos, D, dtype, q, k, v, dout, scale, head, i, dq + head + i * D,
                         dk + head, dv + head, NULL, nb, p, dp, qi, gi);
        }
        free(gi);
        free(qi);
        free(dp);
        free(p);
        free(nb);
    }
    free(pos);
    free(perm);
    return 0;
}

int orc_attention_backward_dq_rows(const orc_spec* s, int64_t B, int64_t H, int64_t D,
                                   int32_t dtype, const void* q, const void* k, const void* v,
                                   const void* dout, double scale, const int64_t* rows,
                                   int64_t nrows, double* dq, int32_t threads) {
    const int64_t N = orc_num_tokens(s);
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    if (orc_order(s, perm) != 0) {
        free(perm);
        return -1;
    }
    int64_t* pos = invert(perm, N);
    int err = 0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        int64_t* nb = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
        double* p = (double*)malloc(sizeof(double) * (size_t)N);
        double* dp = (double*)malloc(sizeof(double) * (size_t)N);
        double* qi = (double*)malloc(sizeof(double) * (size_t)D);
        double* gi = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < B * H * nrows; ++t) {
            const int64_t bh = t / nrows, i = rows[t % nrows];
            double* out = dq + t * D;
            for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
            if (i < 0 || i >= N) {
                err = 1;
                continue;
            }
            grad_row(s, perm, pos, D, dtype, q, k, v, dout, scale, bh * N * D, i, out, NULL, NULL,
                     NULL, nb, p, dp, qi, gi);
        }
        free(gi);
        free(qi);
        free(dp);
        free(p);
        free(nb);
    }
    free(pos);
    free(perm);
    return err ? -2 : 0;
}

/* Does the neighbourhood (either branch) of query i hold a listed key? */
static int attends_listed(const orc_spec* s, const int64_t* perm, const int64_t* pos, int64_t i,
                          const int64_t* slot, int64_t* nb) {
    for (int branch = 0; branch < 2; ++branch) {
        const int64_t n = branch_keys(s, perm, pos, i, branch, nb, NULL);
        for (int64_t a = 0; a < n; ++a)
            if (slot[nb[a]] >= 0) return 1;
    }
    return 0;
}

/* dk and dv of the same gradients for the listed row-major key tokens only.
   dk_j and dv_j sum the terms of every query i whose neighbourhood holds j,
   so each query is tested and those that hold a listed key run the full
   gradient of their row (its softmax and delta need the whole
   neighbourhood); the other queries add nothing.  Per-thread partial sums
   are added at the end. */
int orc_attention_backward_kv_rows(const orc_spec* s, int64_t B, int64_t H, int64_t D,
                                   int32_t dtype, const void* q, const void* k, const void* v,
                                   const void* dout, double scale, const int64_t* keys,
                                   int64_t nkeys, double* dk, double* dv, int32_t threads) {
    const int64_t N = orc_num_tokens(s);
    int64_t* slot = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    for (int64_t j = 0; j < N; ++j) slot[j] = -1;
    for (int64_t a = 0; a < nkeys; ++a) {
        if (keys[a] < 0 || keys[a] >= N || slot[keys[a]] >= 0) {
            free(slot);
            return -2; /* out of range or listed twice */
        }
        slot[keys[a]] = a;
    }
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    if (orc_order(s, perm) != 0) {
        free(perm);
        free(slot);
        return -1;
    }
    int64_t* pos = invert(perm, N);
    const int64_t per_head = nkeys * D;
    for (int64_t t = 0; t < B * H * per_head; ++t) dk[t] = dv[t] = 0.0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        int64_t* nb = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
        double* p = (double*)malloc(sizeof(double) * (size_t)N);
        double* dp = (double*)malloc(sizeof(double) * (size_t)N);
        double* qi = (double*)malloc(sizeof(double) * (size_t)D);
        double* gi = (double*)malloc(sizeof(double) * (size_t)D);
        double* pk = (double*)calloc((size_t)(B * H * per_head), sizeof(double));
        double* pv = (double*)calloc((size_t)(B * H * per_head), sizeof(double));
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < B * H * N; ++t) {
            const int64_t bh = t / N, i = t % N;
            if (!attends_listed(s, perm, pos, i, slot, nb)) continue;
            grad_row(s, perm, pos, D, dtype, q, k, v, dout, scale, bh * N * D, i, NULL,
                     pk + bh * per_head, pv + bh * per_head, slot, nb, p, dp, qi, gi);
        }
#pragma omp critical
        for (int64_t t = 0; t < B * H * per_head; ++t) {
            dk[t] += pk[t];
            dv[t] += pv[t];
        }
        free(pv);
        free(pk);
        free(gi);
        free(qi);
        free(dp);
        free(p);
        free(nb);
    }
    free(pos);
    free(perm);
    free(slot);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Tile classes.                                                            */
/* ------------------------------------------------------------------------ */

/* Every attended pair (i, j) is counted in the cell (tile of the position of
   i, tile of the position of j).  A cell with no pair is empty; one whose
   count equals (valid queries) x (valid keys) of the two tiles is full; any
   other is partial ("Hilbert-Guided Sparse Local Attention", methodology). */
int orc_tile_classes(const orc_spec* s, int64_t q_block, int64_t kv_block, uint8_t* cls,
                     int64_t* pairs, int32_t threads) {
    const int64_t N = orc_num_tokens(s);
    if (q_block < 1 || kv_block < 1) return -1;
    int64_t* perm = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
    if (orc_order(s, perm) != 0) {
        free(perm);
        return -1;
    }
    int64_t* pos = invert(perm, N);
    const int64_t nqt = ceil_div(N, q_block), nkt = ceil_div(N, kv_block);
    int64_t* cnt = (int64_t*)calloc((size_t)(nqt * nkt), sizeof(int64_t));
    int64_t total = 0;
#ifdef _OPENMP
    if (threads > 0) omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel reduction(+ : total)
    {
        int64_t* nb = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t qt = 0; qt < nqt; ++qt) {
            int64_t* row = cnt + qt * nkt;
            for (int64_t p = qt * q_block; p < imin((qt + 1) * q_block, N); ++p) {
                const int64_t n = orc_neighbors(s, perm, pos, perm[p], nb);
                total += n;
                for (int64_t a = 0; a < n; ++a) row[pos[nb[a]] / kv_block] += 1;
                /* the separate variant's partners are attended outside the tile
                   map, but count as attended pairs */
                if (s->skip > 0 && s->skip_mode == ORC_SKIP_SEPARATE)
                    total += orc_partners(s, perm, pos, perm[p], nb);
            }
        }
        free(nb);
    }
    for (int64_t qt = 0; qt < nqt; ++qt) {
        const int64_t nq = imin(q_block, N - qt * q_block);
        for (int64_t kt = 0; kt < nkt; ++kt) {
            const int64_t nk = imin(kv_block, N - kt * kv_block);
            const int64_t c = cnt[qt * nkt + kt];
            cls[qt * nkt + kt] = c == 0 ? 0 : (c == nq * nk ? 2 : 1);
        }
    }
    *pairs = total;
    free(cnt);
    free(pos);
    free(perm);
    return 0;
}
