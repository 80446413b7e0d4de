// Host planner: token order, per-position window boxes, and the exact
// classification of every (query tile, key/value tile) pair into empty,
// partial or full ("Hilbert-Guided Sparse Local Attention", "Methodology in
// Plain English": empty tiles are skipped, partial tiles need element-wise
// masks).  Built once per shape; the result is immutable.
//
// Window rule per pattern dimension (see include/na.h): sliding window of
// `window` positions starting at the (stride-group) centre minus `left`,
// shifted inside the axis (neighbourhood attention, "Generalized Neighborhood
// Attention", abstract) or cut at its ends (band / slide attention,
// "pi-Attention", Eq. 5), on the dilation sub-grid of the query.
#include <algorithm>
#include <cstring>
#include <limits>
#include <string>
#include <unordered_map>

#include "na_internal.h"

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Hilbert order over any rows x cols grid.  The pages give the curve only for
// power-of-two squares (and no orientation); this is the library's reading for
// every grid: blocks are cut the way the classic curve cuts a square (four
// quadrants in a U: near-left travelling across, far-left and far-right
// travelling along, near-right travelling back), blocks more than twice as long
// as wide are cut into two halves along their travel direction instead, and
// the cut points are even wherever possible so that consecutive cells are
// 4-neighbours whenever the block's start and end corners allow it (when they
// cannot, a 3 x 2 end block takes one diagonal step).  On power-of-two squares
// this is exactly the classic curve from (0, 0) to (0, n - 1).
//
// A block is (origin, travel direction a, turn direction b, w cells along a,
// h along b); its walk starts at the origin and ends w - 1 steps along a.
struct CurveBlock {
    int64_t r, c;     // origin cell
    int64_t ar, ac;   // unit travel direction
    int64_t br, bc;   // unit turn direction
    int64_t w, h;
};

int64_t even_cut(int64_t len) {  // even cut near len / 2, in [2, len - 2]
    return std::min(std::max<int64_t>(2 * ((len + 2) / 4), 2), len - 2);
}

void hilbert_order(int64_t rows, int64_t cols, std::vector<int32_t>& perm) {
    perm.clear();
    perm.reserve(rows * cols);
    auto put = [&](int64_t r, int64_t c) { perm.push_back((int32_t)(r * cols + c)); };
    std::vector<CurveBlock> todo;  // processed last-in first-out: children pushed in reverse
    todo.push_back({0, 0, 0, 1, 1, 0, cols, rows});
    while (!todo.empty()) {
        const CurveBlock k = todo.back();
        todo.pop_back();
        if (k.h == 1 || k.w == 1) {
            // a single run; a width-1 block (only a one-column grid) runs along b
            const int64_t n = k.h == 1 ? k.w : k.h;
            const int64_t dr = k.h == 1 ? k.ar : k.br, dc = k.h == 1 ? k.ac : k.bc;
            for (int64_t t = 0; t < n; ++t) put(k.r + t * dr, k.c + t * dc);
            continue;
        }
        if (k.h == 2 && k.w <= 3) {
            // 2 x 2: across, along, back.  3 x 2: across, diagonal back to the
            // second column, then the 2 x 2 pattern.
            put(k.r, k.c);
            put(k.r + k.br, k.c + k.bc);
            int64_t r = k.r + k.ar, c = k.c + k.ac;
            if (k.w == 3) {
                put(r, c);
                put(r + k.br, c + k.bc);
                r += k.ar;
                c += k.ac;
                put(r + k.br, c + k.bc);
                put(r, c);
            } else {
                put(r + k.br, c + k.bc);
                put(r, c);
            }
            continue;
        }
        if (k.h == 2 || k.w > 2 * k.h) {
            const int64_t w1 = even_cut(k.w);
            todo.push_back({k.r + w1 * k.ar, k.c + w1 * k.ac, k.ar, k.ac, k.br, k.bc, k.w - w1, k.h});
            todo.push_back({k.r, k.c, k.ar, k.ac, k.br, k.bc, w1, k.h});
            continue;
        }
        // Quadrants.  Narrow blocks (w <= 3) keep one far row; otherwise the far
        // part is about half the block (no deeper than half its width) and the
        // near part is rounded to an even depth.
        int64_t w1 = k.w - 1, hn = k.h - 1;
        if (k.w > 3) {
            w1 = even_cut(k.w);
            hn = k.h - std::max<int64_t>(1, std::min(k.h / 2, k.w / 2));
            if (hn & 1) hn += (k.h - hn >= 2) ? 1 : -1;
        }
        const int64_t hf = k.h - hn, w2 = k.w - w1;
        // pushed in reverse visiting order
        todo.push_back({k.r + (k.w - 1) * k.ar + (hn - 1) * k.br, k.c + (k.w - 1) * k.ac + (hn - 1) * k.bc,
                        -k.br, -k.bc, -k.ar, -k.ac, hn, w2});
        todo.push_back({k.r + w1 * k.ar + hn * k.br, k.c + w1 * k.ac + hn * k.bc, k.ar, k.ac, k.br, k.bc,
                        w2, hf});
        todo.push_back({k.r + hn * k.br, k.c + hn * k.bc, k.ar, k.ac, k.br, k.bc, w1, hf});
        todo.push_back({k.r, k.c, k.br, k.bc, k.ar, k.ac, hn, w1});
    }
}

struct Axis {
    int64_t L, w, left, stride, dil;
    bool clamp;
    int64_t shift;  // stride-group phase
    bool causal;    // leader = last position of its group (block-causal groups)
};

// [lo, hi) of the keys of coordinate x on one axis, in axis coordinates; with
// dilation only positions congruent to lo modulo dil inside it count.
void axis_window(const Axis& a, int64_t x, int32_t* lo, int32_t* hi) {
    const int64_t g = x % a.dil;
    const int64_t xl = x / a.dil;
    const int64_t Lg = ceil_div(a.L - g, a.dil);
    const int64_t first = ((xl + a.shift) / a.stride) * a.stride - a.shift;
    const int64_t c = first + (a.causal ? a.stride - 1 : a.stride / 2);
    int64_t s, e;
    if (a.clamp) {
        if (a.w >= Lg) {
            s = 0;
            e = Lg;
        } else {
            s = std::min(std::max(c - a.left, int64_t(0)), Lg - a.w);
            e = s + a.w;
        }
    } else {
        s = std::max(c - a.left, int64_t(0));
        e = std::min(c - a.left + a.w, Lg);
    }
    if (e <= s) {
        *lo = 0;
        *hi = 0;
        return;
    }
    *lo = (int32_t)(g + a.dil * s);
    *hi = (int32_t)(g + a.dil * (e - 1) + 1);
}

bool inside(const int32_t* box, const int32_t* c, int pdims, const int32_t* dil) {
    for (int d = 0; d < pdims; ++d) {
        if (c[d] < box[d] || c[d] >= box[3 + d]) return false;
        if (dil[d] > 1 && (c[d] - box[d]) % dil[d] != 0) return false;
    }
    return true;
}

}  // namespace

na_status na_plan_build_host(const na_plan_desc* in, na_plan_s* p) {
    if (!in) {
        na_set_error("descriptor is NULL");
        return NA_ERR_INVALID_ARG;
    }
    na_plan_desc d = *in;
    if (d.ndim < 1 || d.ndim > 3) {
        na_set_error("ndim must be 1, 2 or 3 (got %d)", d.ndim);
        return NA_ERR_INVALID_ARG;
    }
    int64_t N = 1;
    for (int i = 0; i < d.ndim; ++i) {
        if (d.grid[i] < 1) {
            na_set_error("grid[%d] must be >= 1", i);
            return NA_ERR_INVALID_ARG;
        }
        N *= d.grid[i];
    }
    for (int i = d.ndim; i < 3; ++i) d.grid[i] = 1;
    if (N > std::numeric_limits<int32_t>::max() / 2) {
        na_set_error("too many tokens (%lld)", (long long)N);
        return NA_ERR_INVALID_ARG;
    }
    if (d.order < NA_ORDER_ROW_MAJOR || d.order > NA_ORDER_HILBERT) {
        na_set_error("unknown order %d", d.order);
        return NA_ERR_INVALID_ARG;
    }
    if (d.dtype != NA_BF16 && d.dtype != NA_F32) {
        na_set_error("unknown dtype %d", d.dtype);
        return NA_ERR_INVALID_ARG;
    }
    if (d.head_dim < 1) {
        na_set_error("head_dim must be >= 1");
        return NA_ERR_INVALID_ARG;
    }
    // Default query tile: at head_dim 128 each key/value tile carries twice the
    // MFMA work per byte staged, so eight waves (256 queries) share one tile.
    if (d.q_block == 0)
        d.q_block = d.dtype == NA_F32 ? NA_Q_BLOCK_F32 : (d.head_dim >= 128 ? 256 : 128);
    if (d.kv_block == 0) d.kv_block = d.dtype == NA_F32 ? NA_KV_BLOCK_F32 : NA_KV_BLOCK_BF16;
    if (d.q_block < 1 || d.kv_block < 1) {
        na_set_error("q_block and kv_block must be >= 1");
        return NA_ERR_INVALID_ARG;
    }
    const int pdims = d.order == NA_ORDER_HILBERT ? 1 : d.ndim;
    if (d.order == NA_ORDER_HILBERT && d.ndim != 2) {
        na_set_error("Hilbert order needs a 2-D grid");
        return NA_ERR_UNSUPPORTED;
    }
    if (d.order == NA_ORDER_TILED) {
        for (int i = 0; i < d.ndim; ++i)
            if (d.tile[i] < 1) {
                na_set_error("tile[%d] must be >= 1", i);
                return NA_ERR_INVALID_ARG;
            }
        for (int i = d.ndim; i < 3; ++i) d.tile[i] = 1;
    }
    Axis ax[3];
    for (int i = 0; i < 3; ++i) {
        if (i >= pdims) {
            ax[i] = Axis{1, 1, 0, 1, 1, true, 0, false};
            p->plen[i] = 1;
            p->left[i] = 0;
            p->clamp[i] = 1;
            d.window[i] = 1;
            d.window_left[i] = 0;
            d.stride[i] = 1;
            d.shift[i] = 0;
            d.dilation[i] = 1;
            d.causal[i] = 0;
            d.boundary[i] = NA_BOUND_CLAMP;
            continue;
        }
        const int64_t L = d.order == NA_ORDER_HILBERT ? N : d.grid[i];
        if (d.window[i] < 1 || d.stride[i] < 1 || d.dilation[i] < 1) {
            na_set_error("window, stride and dilation of dimension %d must be >= 1", i);
            return NA_ERR_INVALID_ARG;
        }
        if (d.stride[i] > d.window[i]) {
            // a group wider than its window would not see all of itself
            na_set_error("stride[%d] (%d) must not exceed window[%d] (%d)", i, d.stride[i], i,
                         d.window[i]);
            return NA_ERR_INVALID_ARG;
        }
        if (d.shift[i] < 0 || d.shift[i] >= d.stride[i]) {
            na_set_error("shift[%d] (%d) must lie in [0, stride[%d])", i, d.shift[i], i);
            return NA_ERR_INVALID_ARG;
        }
        if (d.causal[i] != 0 && d.causal[i] != 1) {
            na_set_error("causal[%d] must be 0 or 1", i);
            return NA_ERR_INVALID_ARG;
        }
        if (d.boundary[i] != NA_BOUND_CLAMP && d.boundary[i] != NA_BOUND_TRUNCATE) {
            na_set_error("boundary[%d] must be NA_BOUND_CLAMP or NA_BOUND_TRUNCATE", i);
            return NA_ERR_INVALID_ARG;
        }
        int64_t left = d.window_left[i];
        if (d.causal[i]) {
            left = d.window[i] - 1;
            d.boundary[i] = NA_BOUND_TRUNCATE;
        } else if (left < 0) {
            if (left != -1) {
                na_set_error("window_left[%d] must be >= 0 or -1", i);
                return NA_ERR_INVALID_ARG;
            }
            left = d.window[i] / 2;
        }
        d.window_left[i] = (int32_t)left;
        ax[i] = Axis{L, d.window[i], left, d.stride[i], d.dilation[i],
                     d.boundary[i] == NA_BOUND_CLAMP, d.shift[i], d.causal[i] != 0};
        p->plen[i] = (int32_t)L;
        p->left[i] = (int32_t)left;
        p->clamp[i] = d.boundary[i] == NA_BOUND_CLAMP;
        if (d.dilation[i] > 1) p->has_dilation = true;
    }
    // pi-Attention partner
    if (d.skip < 0 || (d.skip_both != 0 && d.skip_both != 1) || d.skip_mode < NA_SKIP_UNION ||
        d.skip_mode > NA_SKIP_SEPARATE) {
        na_set_error("skip must be >= 0, skip_both 0 or 1, skip_mode an NA_SKIP_* value");
        return NA_ERR_INVALID_ARG;
    }
    if (d.skip > 0 && pdims != 1) {
        na_set_error("the skip partner is defined on one pattern dimension (1-D grids, Hilbert order)");
        return NA_ERR_UNSUPPORTED;
    }
    if (d.skip > 0 && d.skip_mode == NA_SKIP_FIXED_FUSION &&
        !(d.skip_prior > 0.f && d.skip_prior < 1.f)) {
        na_set_error("skip_prior must lie in (0, 1) for fixed fusion");
        return NA_ERR_INVALID_ARG;
    }
    if (d.skip == 0) {
        d.skip_both = 0;
        d.skip_mode = NA_SKIP_UNION;
        d.skip_prior = 0.f;
    }
    if (d.skip_mode != NA_SKIP_FIXED_FUSION) d.skip_prior = 0.f;
    p->partner_union = d.skip > 0 && d.skip_mode != NA_SKIP_SEPARATE;
    p->desc = d;
    p->n_tokens = N;
    p->pdims = pdims;

    // ---- token order ----------------------------------------------------
    p->perm.resize(N);
    if (d.order == NA_ORDER_ROW_MAJOR) {
        for (int64_t i = 0; i < N; ++i) p->perm[i] = (int32_t)i;
        p->identity_order = true;
    } else if (d.order == NA_ORDER_HILBERT) {
        hilbert_order(d.grid[0], d.grid[1], p->perm);
        p->identity_order = true;  // a one-row or one-column grid
        for (int64_t i = 0; i < N; ++i)
            if (p->perm[i] != i) {
                p->identity_order = false;
                break;
            }
    } else {
        const int64_t g1 = d.grid[1], g2 = d.grid[2];
        const int64_t nt0 = ceil_div(d.grid[0], d.tile[0]);
        const int64_t nt1 = ceil_div(g1, d.tile[1]);
        const int64_t nt2 = ceil_div(g2, d.tile[2]);
        int64_t pos = 0;
        for (int64_t a = 0; a < nt0; ++a)
            for (int64_t b = 0; b < nt1; ++b)
                for (int64_t c = 0; c < nt2; ++c) {
                    const int64_t x0 = a * d.tile[0], x1 = std::min<int64_t>(x0 + d.tile[0], d.grid[0]);
                    const int64_t y0 = b * d.tile[1], y1 = std::min<int64_t>(y0 + d.tile[1], g1);
                    const int64_t z0 = c * d.tile[2], z1 = std::min<int64_t>(z0 + d.tile[2], g2);
                    for (int64_t x = x0; x < x1; ++x)
                        for (int64_t y = y0; y < y1; ++y)
                            for (int64_t z = z0; z < z1; ++z)
                                p->perm[pos++] = (int32_t)((x * g1 + y) * g2 + z);
                }
        p->identity_order = true;
        for (int64_t i = 0; i < N; ++i)
            if (p->perm[i] != i) {
                p->identity_order = false;
                break;
            }
    }

    // ---- pattern coordinates and window boxes per sequence position ------
    p->kcoord.assign(N * 4, 0);
    p->qbox.assign(N * 8, 0);
    int64_t pairs = 0;
    for (int64_t pos = 0; pos < N; ++pos) {
        int32_t* c = &p->kcoord[pos * 4];
        if (d.order == NA_ORDER_HILBERT) {
            c[0] = (int32_t)pos;
        } else {
            const int64_t tok = p->perm[pos];
            c[0] = (int32_t)(tok / ((int64_t)d.grid[1] * d.grid[2]));
            c[1] = (int32_t)((tok / d.grid[2]) % d.grid[1]);
            c[2] = (int32_t)(tok % d.grid[2]);
        }
        int32_t* box = &p->qbox[pos * 8];
        int64_t cnt = 1;
        for (int i = 0; i < 3; ++i) {
            axis_window(ax[i], c[i], &box[i], &box[3 + i]);
            const int64_t span = box[3 + i] - box[i];
            cnt *= span <= 0 ? 0 : ceil_div(span, ax[i].dil);
        }
        pairs += cnt;
    }
    // One pattern dimension: the pattern coordinate of a position is the
    // position itself (1-D grids in either order, and the curve position of the
    // Hilbert order), so partners are positions pos -/+ skip.
    const int64_t skip = d.skip;
    auto is_partner = [&](int64_t qp, int64_t kp) {
        return skip > 0 && (kp == qp - skip || (d.skip_both && kp == qp + skip));
    };
    const int32_t dil1[3] = {(int32_t)ax[0].dil, 1, 1};
    if (skip > 0) {
        for (int64_t pos = 0; pos < N; ++pos) {
            for (int t = 0; t < 1 + d.skip_both; ++t) {
                const int64_t y = t == 0 ? pos - skip : pos + skip;
                if (y < 0 || y >= N) continue;
                // a partner inside the window adds nothing to the union
                if (!p->partner_union || !inside(&p->qbox[pos * 8], &p->kcoord[y * 4], 1, dil1))
                    ++pairs;
            }
        }
    }

    // ---- tile classification ---------------------------------------------
    const int64_t qb = d.q_block, kb = d.kv_block;
    const int64_t nqt = ceil_div(N, qb), nkt = ceil_div(N, kb);
    int32_t dil[3] = {(int32_t)ax[0].dil, (int32_t)ax[1].dil, (int32_t)ax[2].dil};
    // key bounding boxes of the key/value tiles
    std::vector<int32_t> kbox(nkt * 6);
    for (int64_t t = 0; t < nkt; ++t) {
        int32_t* b = &kbox[t * 6];
        for (int i = 0; i < 3; ++i) {
            b[i] = std::numeric_limits<int32_t>::max();
            b[3 + i] = std::numeric_limits<int32_t>::min();
        }
        for (int64_t pos = t * kb; pos < std::min(N, (t + 1) * kb); ++pos)
            for (int i = 0; i < 3; ++i) {
                b[i] = std::min(b[i], p->kcoord[pos * 4 + i]);
                b[3 + i] = std::max(b[3 + i], p->kcoord[pos * 4 + i] + 1);
            }
    }
    p->row_ptr.assign(nqt + 1, 0);
    p->entries.clear();
    int64_t n_partial = 0, n_full = 0;
    for (int64_t qt = 0; qt < nqt; ++qt) {
        const int64_t q0 = qt * qb, q1 = std::min(N, q0 + qb);
        // intersection and union of the query boxes of this tile
        int32_t ilo[3], ihi[3], ulo[3], uhi[3];
        for (int i = 0; i < 3; ++i) {
            ilo[i] = std::numeric_limits<int32_t>::min();
            ihi[i] = std::numeric_limits<int32_t>::max();
            ulo[i] = std::numeric_limits<int32_t>::max();
            uhi[i] = std::numeric_limits<int32_t>::min();
        }
        bool any_empty_query = false;
        for (int64_t pos = q0; pos < q1; ++pos) {
            const int32_t* box = &p->qbox[pos * 8];
            bool empty = false;
            for (int i = 0; i < 3; ++i) empty |= box[3 + i] <= box[i];
            if (empty) {
                any_empty_query = true;
                continue;
            }
            for (int i = 0; i < 3; ++i) {
                ilo[i] = std::max(ilo[i], box[i]);
                ihi[i] = std::min(ihi[i], box[3 + i]);
                ulo[i] = std::min(ulo[i], box[i]);
                uhi[i] = std::max(uhi[i], box[3 + i]);
            }
        }
        for (int64_t kt = 0; kt < nkt; ++kt) {
            const int32_t* kbx = &kbox[kt * 6];
            bool disjoint = false;
            for (int i = 0; i < p->pdims; ++i)
                disjoint |= kbx[3 + i] <= ulo[i] || kbx[i] >= uhi[i];
            // partners of this query tile: positions [q0, q1) shifted by -/+ skip
            bool partners_here = false;
            if (p->partner_union) {
                const int64_t k0 = kt * kb, k1 = std::min(N, k0 + kb);
                partners_here = q0 - skip < k1 && q1 - skip > k0;
                if (d.skip_both) partners_here |= q0 + skip < k1 && q1 + skip > k0;
            }
            if (disjoint && !partners_here) continue;  // empty (also when every query is empty)
            bool full = !disjoint && !any_empty_query && !p->has_dilation;
            for (int i = 0; full && i < p->pdims; ++i)
                full = ilo[i] <= kbx[i] && kbx[3 + i] <= ihi[i];
            int cls = 2;
            if (!full) {
                // exact: look for both an attended and an unattended pair
                bool hit = false, miss = false;
                const int64_t k0 = kt * kb, k1 = std::min(N, k0 + kb);
                for (int64_t qp = q0; qp < q1 && !(hit && miss); ++qp)
                    for (int64_t kp = k0; kp < k1; ++kp) {
                        if (inside(&p->qbox[qp * 8], &p->kcoord[kp * 4], p->pdims, dil) ||
                            (p->partner_union && is_partner(qp, kp)))
                            hit = true;
                        else
                            miss = true;
                        if (hit && miss) break;
                    }
                if (!hit) continue;
                cls = miss ? 1 : 2;
            }
            if (cls == 1)
                ++n_partial;
            else
                ++n_full;
            p->entries.push_back(NaEntry{(int32_t)kt, -1});
            p->entry_cls.push_back((uint8_t)cls);
        }
        p->row_ptr[qt + 1] = (int32_t)p->entries.size();
    }

    // ---- element masks of partial tiles and of tiles past the last key ------
    // Bit (row r, key k) of a tile mask: query position q0 + r and key position
    // k0 + k are both valid tokens and the key lies in the query's window.
    // Identical masks are stored once.
    const int kvw = (int)ceil_div(kb, 32);
    p->mask_words = kvw;
    p->masks.clear();
    // With fixed fusion a second plane (same id) marks the partners outside
    // the window; a tile holding any of them always carries a mask.
    const bool fusion = p->partner_union && d.skip_mode == NA_SKIP_FIXED_FUSION;
    p->skip_masks.clear();
    std::unordered_map<std::string, int32_t> seen;
    std::vector<uint32_t> m((size_t)(qb * kvw)), sk((size_t)(qb * kvw));
    for (int64_t qt = 0; qt < nqt; ++qt) {
        for (int32_t e = p->row_ptr[qt]; e < p->row_ptr[qt + 1]; ++e) {
            const int64_t kt = p->entries[e].kt;
            const bool full = p->entry_cls[e] == 2;
            const bool last = (kt + 1) * kb > N;
            if (full && !last && !fusion) continue;  // no mask needed
            std::fill(m.begin(), m.end(), 0u);
            std::fill(sk.begin(), sk.end(), 0u);
            bool any_skip = false;
            for (int64_t r = 0; r < qb; ++r) {
                const int64_t qp = qt * qb + r;
                if (qp >= N) break;
                for (int64_t k = 0; k < kb; ++k) {
                    const int64_t kp = kt * kb + k;
                    if (kp >= N) break;
                    const bool in = inside(&p->qbox[qp * 8], &p->kcoord[kp * 4], p->pdims, dil);
                    const bool part = p->partner_union && is_partner(qp, kp);
                    if (full || in || part) m[r * kvw + k / 32] |= 1u << (k % 32);
                    if (fusion && part && !in) {
                        sk[r * kvw + k / 32] |= 1u << (k % 32);
                        any_skip = true;
                    }
                }
            }
            if (full && !last && !any_skip) continue;
            std::string key((const char*)m.data(), m.size() * sizeof(uint32_t));
            if (fusion) key.append((const char*)sk.data(), sk.size() * sizeof(uint32_t));
            auto it = seen.find(key);
            int32_t id;
            if (it == seen.end()) {
                id = (int32_t)seen.size();
                seen.emplace(std::move(key), id);
                p->masks.insert(p->masks.end(), m.begin(), m.end());
                if (fusion) p->skip_masks.insert(p->skip_masks.end(), sk.begin(), sk.end());
            } else {
                id = it->second;
            }
            p->entries[e].mask = id;
        }
    }
    p->n_masks = (int64_t)seen.size();

    // ---- walk order inside a row -----------------------------------------------
    // A row whose key/value tiles are consecutive (bands, causal windows) is
    // stored rotated: it starts at its tile whose index is a multiple of the
    // row length and wraps around.  Neighbouring query tiles, whose rows
    // overlap, then stage the same key/value tile at the same step of their
    // walks, so workgroups running at the same time share it in L2.  The
    // kernels' online softmax takes a row's tiles in any order; rows of other
    // shapes stay ascending.
    for (int64_t qt = 0; qt < nqt; ++qt) {
        const int32_t r0 = p->row_ptr[qt], r1 = p->row_ptr[qt + 1];
        const int32_t len = r1 - r0;
        if (len < 2 || p->entries[r1 - 1].kt - p->entries[r0].kt != len - 1) continue;
        const int32_t j0 = (len - p->entries[r0].kt % len) % len;
        std::rotate(p->entries.begin() + r0, p->entries.begin() + r0 + j0, p->entries.begin() + r1);
        std::rotate(p->entry_cls.begin() + r0, p->entry_cls.begin() + r0 + j0, p->entry_cls.begin() + r1);
    }

    // ---- the same map by key/value tile --------------------------------------
    p->t_row_ptr.assign(nkt + 1, 0);
    for (const NaEntry& e : p->entries) ++p->t_row_ptr[e.kt + 1];
    for (int64_t kt = 0; kt < nkt; ++kt) p->t_row_ptr[kt + 1] += p->t_row_ptr[kt];
    p->t_entries.assign(p->entries.size(), NaEntry{0, -1});
    {
        std::vector<int32_t> fill(p->t_row_ptr.begin(), p->t_row_ptr.end() - 1);
        for (int64_t qt = 0; qt < nqt; ++qt)
            for (int32_t e = p->row_ptr[qt]; e < p->row_ptr[qt + 1]; ++e)
                p->t_entries[fill[p->entries[e].kt]++] = NaEntry{(int32_t)qt, p->entries[e].mask};
    }
    // ---- key/value tiles in pairs: merge the two ascending query-tile lists --
    {
        const int64_t npair = ceil_div(nkt, 2);
        p->p_row_ptr.assign(npair + 1, 0);
        p->p_entries.clear();
        for (int64_t g = 0; g < npair; ++g) {
            const int64_t ka = 2 * g, kb2 = 2 * g + 1;
            int32_t a = p->t_row_ptr[ka], ae = p->t_row_ptr[ka + 1];
            int32_t c = kb2 < nkt ? p->t_row_ptr[kb2] : 0, ce = kb2 < nkt ? p->t_row_ptr[kb2 + 1] : 0;
            while (a < ae || c < ce) {
                const int32_t qa = a < ae ? p->t_entries[a].kt : std::numeric_limits<int32_t>::max();
                const int32_t qc = c < ce ? p->t_entries[c].kt : std::numeric_limits<int32_t>::max();
                const int32_t qt = std::min(qa, qc);
                NaPairEntry en{qt, NA_MASK_NONE, NA_MASK_NONE, 0};
                if (qa == qt) en.mask0 = p->t_entries[a++].mask;
                if (qc == qt) en.mask1 = p->t_entries[c++].mask;
                p->p_entries.push_back(en);
            }
            p->p_row_ptr[g + 1] = (int32_t)p->p_entries.size();
        }
    }
    // ---- dispatch order of the query tiles ----------------------------------------
    // A one-dimensional map whose first walk is shorter than its last (a causal
    // window: the walks grow from the start of the sequence) runs its query
    // tiles in descending order, longest walks first.  Maps in more dimensions
    // keep ascending order, which measured faster on the tiled windows.
    p->q_desc = p->pdims == 1 && nqt > 1 &&
                p->row_ptr[1] - p->row_ptr[0] < p->row_ptr[nqt] - p->row_ptr[nqt - 1];
    p->stats.n_tokens = N;
    p->stats.q_block = qb;
    p->stats.kv_block = kb;
    p->stats.n_q_tiles = nqt;
    p->stats.n_kv_tiles = nkt;
    p->stats.n_partial = n_partial;
    p->stats.n_full = n_full;
    p->stats.n_empty = nqt * nkt - n_partial - n_full;
    p->stats.attended_pairs = pairs;
    return NA_OK;
}
