// C ABI of libna.so: plan lifetime, validation, device upload and kernel
// dispatch.  Every entry point returns an na_status and never throws; all
// argument checks run on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <chrono>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <new>

#include "na_internal.h"

namespace {
thread_local char g_err[512] = "";

// NA_LOG=1 prints each plan's statistics to stderr when it is created;
// NA_LOG=2 also prints every forward launch's grid and split.  Read once.
int log_level() {
    static const int level = [] {
        const char* v = std::getenv("NA_LOG");
        return v ? std::atoi(v) : 0;
    }();
    return level;
}

const char* hip_err(hipError_t e) { return hipGetErrorString(e); }

template <typename T>
na_status upload(const std::vector<T>& host, T** dev) {
    *dev = nullptr;
    if (host.empty()) return NA_OK;
    const size_t bytes = host.size() * sizeof(T);
    hipError_t e = hipMalloc((void**)dev, bytes);
    if (e != hipSuccess) {
        *dev = nullptr;
        na_set_error("hipMalloc(%zu) failed: %s", bytes, hip_err(e));
        return e == hipErrorOutOfMemory ? NA_ERR_OUT_OF_MEMORY : NA_ERR_DEVICE;
    }
    e = hipMemcpy(*dev, host.data(), bytes, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        na_set_error("hipMemcpy(%zu) failed: %s", bytes, hip_err(e));
        return NA_ERR_DEVICE;
    }
    return NA_OK;
}

void free_device(na_plan_s* p) {
    if (!p->on_device) return;
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != p->device) (void)hipSetDevice(p->device);
    (void)hipFree(p->d_perm);
    (void)hipFree(p->d_row_ptr);
    (void)hipFree(p->d_entries);
    (void)hipFree(p->d_t_row_ptr);
    (void)hipFree(p->d_t_entries);
    (void)hipFree(p->d_p_row_ptr);
    (void)hipFree(p->d_p_entries);
    (void)hipFree(p->d_masks);
    (void)hipFree(p->d_skip_masks);
    (void)hipFree(p->d_zero);
    if (cur != p->device && cur >= 0) (void)hipSetDevice(cur);
    p->d_perm = nullptr;
    p->d_row_ptr = nullptr;
    p->d_entries = nullptr;
    p->d_t_row_ptr = nullptr;
    p->d_t_entries = nullptr;
    p->d_p_row_ptr = nullptr;
    p->d_p_entries = nullptr;
    p->d_masks = nullptr;
    p->d_skip_masks = nullptr;
    p->d_zero = nullptr;
    p->on_device = false;
}

int elem_bytes(const na_plan_s* p) { return p->desc.dtype == NA_F32 ? 4 : 2; }

// Validate one [B, H, N, D] tensor view against the plan.
na_status check_tensor(const na_plan_s* p, const na_tensor* t, const char* name, int64_t B,
                       int64_t H) {
    if (!t || !t->ptr) {
        na_set_error("%s is NULL", name);
        return NA_ERR_INVALID_ARG;
    }
    const int64_t D = p->desc.head_dim;
    const int64_t align = 16 / elem_bytes(p);  // elements per 16 bytes
    if (((uintptr_t)t->ptr) % 16 != 0) {
        na_set_error("%s must be 16-byte aligned", name);
        return NA_ERR_INVALID_ARG;
    }
    if (t->stride_n < D || t->stride_n % align != 0 || t->stride_h % align != 0 ||
        t->stride_b % align != 0 || t->stride_h < 0 || t->stride_b < 0) {
        na_set_error("%s strides (b=%lld h=%lld n=%lld) must be non-negative multiples of %lld "
                     "with stride_n >= head_dim",
                     name, (long long)t->stride_b, (long long)t->stride_h, (long long)t->stride_n,
                     (long long)align);
        return NA_ERR_INVALID_ARG;
    }
    (void)B;
    (void)H;
    // element offsets inside one (batch, head) slice must fit in 31 bits
    if ((p->n_tokens - 1) * t->stride_n + D > 0x7fffffff) {
        na_set_error("%s: a (batch, head) slice spans more than 2^31 elements", name);
        return NA_ERR_UNSUPPORTED;
    }
    return NA_OK;
}


size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Bytes of the permute passes' buffers (gathered q, k, v, out and lse).
size_t permute_ws_bytes(const na_plan_s* p, int64_t B, int64_t H, uint32_t flags) {
    if (!(flags & NA_FWD_PERMUTE_PASSES) || p->identity_order) return 0;
    const size_t rows = (size_t)B * (size_t)H * (size_t)p->n_tokens;
    const size_t t = rows * (size_t)p->desc.head_dim * (size_t)elem_bytes(p);
    return 4 * up256(t) + up256(rows * sizeof(float));
}

// The split tail cuts a tail tile into at most kMaxShares shares, and all
// shares together fill at most kShareRounds resident rounds.
constexpr int64_t kMaxShares = 16;
constexpr int64_t kShareRounds = 4;

// Bytes of the split tail's shares: at most kShareRounds * split_capacity of
// them, each q_block rows of head_dim fp32 values plus two floats.
size_t split_ws_bytes(const na_plan_s* p, uint32_t flags) {
    if (!(flags & NA_FWD_SPLIT_TAIL) || p->split_capacity <= 0) return 0;
    const size_t rows = (size_t)(kShareRounds * p->split_capacity) * (size_t)p->desc.q_block;
    return up256(rows * (size_t)p->desc.head_dim * sizeof(float)) + up256(rows * 2 * sizeof(float));
}

}  // namespace

void na_set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

extern "C" {

const char* na_last_error(void) { return g_err; }

int32_t na_abi_version(void) { return NA_ABI_VERSION; }

const char* na_status_string(na_status s) {
    switch (s) {
        case NA_OK: return "ok";
        case NA_ERR_INVALID_ARG: return "invalid argument";
        case NA_ERR_UNSUPPORTED: return "unsupported";
        case NA_ERR_OUT_OF_MEMORY: return "out of memory";
        case NA_ERR_DEVICE: return "device error";
        case NA_ERR_PLAN_MISMATCH: return "plan mismatch";
    }
    return "unknown status";
}

na_status na_plan_create(const na_plan_desc* desc, uint32_t flags, na_plan_t* out) {
    if (!out) {
        na_set_error("plan output pointer is NULL");
        return NA_ERR_INVALID_ARG;
    }
    *out = nullptr;
    if (flags & ~NA_PLAN_HOST_ONLY) {
        na_set_error("unknown plan flags 0x%x", flags);
        return NA_ERR_INVALID_ARG;
    }
    const auto t_start = std::chrono::steady_clock::now();
    na_plan_s* p = new (std::nothrow) na_plan_s();
    if (!p) {
        na_set_error("host allocation failed");
        return NA_ERR_OUT_OF_MEMORY;
    }
    na_status st;
    try {
        st = na_plan_build_host(desc, p);
    } catch (const std::bad_alloc&) {
        na_set_error("host allocation failed while planning");
        st = NA_ERR_OUT_OF_MEMORY;
    }
    if (st != NA_OK) {
        delete p;
        return st;
    }
    if (!(flags & NA_PLAN_HOST_ONLY)) {
        hipError_t e = hipGetDevice(&p->device);
        if (e != hipSuccess) {
            na_set_error("hipGetDevice failed: %s", hip_err(e));
            delete p;
            return NA_ERR_DEVICE;
        }
        p->on_device = true;
        const std::vector<int32_t> none;
        st = upload(p->identity_order ? none : p->perm, &p->d_perm);
        if (st == NA_OK) st = upload(p->row_ptr, &p->d_row_ptr);
        if (st == NA_OK) st = upload(p->entries, &p->d_entries);
        if (st == NA_OK) st = upload(p->t_row_ptr, &p->d_t_row_ptr);
        if (st == NA_OK) st = upload(p->t_entries, &p->d_t_entries);
        if (st == NA_OK) st = upload(p->p_row_ptr, &p->d_p_row_ptr);
        if (st == NA_OK) st = upload(p->p_entries, &p->d_p_entries);
        if (st == NA_OK) st = upload(p->masks, &p->d_masks);
        if (st == NA_OK) st = upload(p->skip_masks, &p->d_skip_masks);
        if (st == NA_OK) {
            const std::vector<uint8_t> zeros(1024, 0);
            st = upload(zeros, (uint8_t**)&p->d_zero);
        }
        if (st != NA_OK) {
            free_device(p);
            delete p;
            return st;
        }
        // the split tail runs on the bf16 kernels without the fixed-fusion
        // bias and without the separate softmax's partner branch in their
        // epilogue (the 32-query-per-wave kernels fuse it; at q_block 192 and
        // 384 it is a second kernel after the merge)
        const na_plan_desc& d = p->desc;
        const bool sep_in_epilogue = d.skip > 0 && d.skip_mode == NA_SKIP_SEPARATE &&
                                     d.q_block != 192 && d.q_block != 384;
        p->split_capacity = sep_in_epilogue ? 0 : na_attn_split_capacity(
            d.dtype, d.head_dim, d.q_block, d.skip > 0 && d.skip_mode == NA_SKIP_FIXED_FUSION);
        p->stats.resident_workgroups = p->split_capacity;
    }
    for (size_t t = 0; t + 1 < p->row_ptr.size(); ++t)
        p->max_row_len = std::max(p->max_row_len, p->row_ptr[t + 1] - p->row_ptr[t]);
    if (log_level() >= 1) {
        const double ms =
            std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t_start)
                .count();
        const na_plan_stats& st = p->stats;
        std::fprintf(stderr,
                     "na: plan N=%lld order=%d head_dim=%d dtype=%d q_block=%lld kv_block=%lld "
                     "tiles=%lldx%lld empty=%lld partial=%lld full=%lld masks=%lld "
                     "pairs_per_head=%lld max_row=%d resident_workgroups=%lld tile_order=%s %s %.2f ms\n",
                     (long long)st.n_tokens, p->desc.order, p->desc.head_dim, p->desc.dtype,
                     (long long)st.q_block, (long long)st.kv_block, (long long)st.n_q_tiles,
                     (long long)st.n_kv_tiles, (long long)st.n_empty, (long long)st.n_partial,
                     (long long)st.n_full, (long long)p->n_masks, (long long)st.attended_pairs,
                     p->max_row_len, (long long)st.resident_workgroups,
                     p->q_desc ? "descending" : "ascending", p->on_device ? "device" : "host-only", ms);
    }
    *out = p;
    return NA_OK;
}

na_status na_plan_destroy(na_plan_t p) {
    if (!p) return NA_OK;
    free_device(p);
    delete p;
    return NA_OK;
}

na_status na_plan_get_stats(na_plan_t p, na_plan_stats* s) {
    if (!p || !s) {
        na_set_error("plan or stats pointer is NULL");
        return NA_ERR_INVALID_ARG;
    }
    *s = p->stats;
    return NA_OK;
}

na_status na_plan_get_bounds(na_plan_t p, na_plan_bounds* out) {
    if (!p || !out) {
        na_set_error("plan or bounds pointer is NULL");
        return NA_ERR_INVALID_ARG;
    }
    const int64_t N = p->stats.n_tokens, qb = p->stats.q_block, kb = p->stats.kv_block;
    const int64_t nq = p->stats.n_q_tiles, nk = p->stats.n_kv_tiles;
    const int64_t visited = p->stats.n_partial + p->stats.n_full;
    const int64_t pairs = p->stats.attended_pairs;
    // token pairs inside the visited tiles, ragged last tiles at their true size
    int64_t inside = 0;
    for (int64_t qt = 0; qt < nq; ++qt) {
        const int64_t qs = std::min(qb, N - qt * qb);
        for (int32_t e = p->row_ptr[qt]; e < p->row_ptr[qt + 1]; ++e)
            inside += qs * std::min(kb, N - (int64_t)p->entries[e].kt * kb);
    }
    const double inf = std::numeric_limits<double>::infinity();
    out->flop = pairs > 0 ? (double)N * (double)N / (double)pairs : inf;
    out->tile = visited > 0 ? (double)nq * (double)nk / (double)visited : inf;
    out->useful_fraction = inside > 0 ? (double)pairs / (double)inside : 1.0;
    return NA_OK;
}

na_status na_plan_get_classes(na_plan_t p, uint8_t* host, size_t n) {
    if (!p || !host) {
        na_set_error("plan or output pointer is NULL");
        return NA_ERR_INVALID_ARG;
    }
    const int64_t nq = p->stats.n_q_tiles, nk = p->stats.n_kv_tiles;
    if ((int64_t)n < nq * nk) {
        na_set_error("class buffer holds %zu entries, need %lld", n, (long long)(nq * nk));
        return NA_ERR_INVALID_ARG;
    }
    std::memset(host, 0, (size_t)(nq * nk));
    for (int64_t qt = 0; qt < nq; ++qt)
        for (int32_t e = p->row_ptr[qt]; e < p->row_ptr[qt + 1]; ++e)
            host[qt * nk + p->entries[e].kt] = p->entry_cls[e];
    return NA_OK;
}

na_status na_plan_get_order(na_plan_t p, int32_t* host, size_t n) {
    if (!p || !host) {
        na_set_error("plan or output pointer is NULL");
        return NA_ERR_INVALID_ARG;
    }
    if ((int64_t)n < p->n_tokens) {
        na_set_error("order buffer holds %zu entries, need %lld", n, (long long)p->n_tokens);
        return NA_ERR_INVALID_ARG;
    }
    std::memcpy(host, p->perm.data(), sizeof(int32_t) * (size_t)p->n_tokens);
    return NA_OK;
}

size_t na_forward_workspace_bytes(na_plan_t p, int64_t B, int64_t H, uint32_t flags) {
    if (!p || B < 1 || H < 1) return 0;
    return permute_ws_bytes(p, B, H, flags) + split_ws_bytes(p, flags);
}

na_status na_forward(na_plan_t p, int64_t B, int64_t H, const na_tensor* q, const na_tensor* k,
                     const na_tensor* v, const na_tensor* out, float* lse, float scale,
                     uint32_t flags, void* workspace, size_t ws_bytes, void* stream) {
    if (!p) {
        na_set_error("plan is NULL");
        return NA_ERR_INVALID_ARG;
    }
    if (!p->on_device) {
        na_set_error("plan was built host-only and cannot run");
        return NA_ERR_PLAN_MISMATCH;
    }
    if (flags & ~(NA_FWD_PERMUTE_PASSES | NA_FWD_SPLIT_TAIL)) {
        na_set_error("unknown forward flags 0x%x", flags);
        return NA_ERR_INVALID_ARG;
    }
    if (B < 1 || H < 1) {
        na_set_error("B and H must be >= 1");
        return NA_ERR_INVALID_ARG;
    }
    const int64_t n_wg = p->stats.n_q_tiles * B * H;
    if (n_wg > 0x7fffffff || B * H > 0x7fffffff / (p->n_tokens > 0 ? p->n_tokens : 1)) {
        na_set_error("B * H * tiles too large");
        return NA_ERR_INVALID_ARG;
    }
    na_status st;
    if ((st = check_tensor(p, q, "q", B, H)) != NA_OK) return st;
    if ((st = check_tensor(p, k, "k", B, H)) != NA_OK) return st;
    if ((st = check_tensor(p, v, "v", B, H)) != NA_OK) return st;
    if ((st = check_tensor(p, out, "out", B, H)) != NA_OK) return st;
    if (lse && ((uintptr_t)lse) % 4 != 0) {
        na_set_error("lse must be 4-byte aligned");
        return NA_ERR_INVALID_ARG;
    }
    if (!(scale > 0.f) || scale == __builtin_inff()) {
        na_set_error("scale must be finite and positive");
        return NA_ERR_INVALID_ARG;
    }
    const na_plan_desc& d = p->desc;
    const bool fusion = d.skip > 0 && d.skip_mode == NA_SKIP_FIXED_FUSION;
    const bool separate = d.skip > 0 && d.skip_mode == NA_SKIP_SEPARATE;
    if (!na_attn_supported(d.dtype, d.head_dim, d.q_block, d.kv_block, fusion)) {
        na_set_error("no kernel for dtype=%d head_dim=%d q_block=%d kv_block=%d%s", d.dtype,
                     d.head_dim, d.q_block, d.kv_block, fusion ? " with fixed fusion" : "");
        return NA_ERR_UNSUPPORTED;
    }
    if (separate && !na_skip_supported(d.dtype, d.head_dim)) {
        na_set_error("no partner-branch kernel for dtype=%d head_dim=%d", d.dtype, d.head_dim);
        return NA_ERR_UNSUPPORTED;
    }
    int cur = -1;
    hipError_t he = hipGetDevice(&cur);
    if (he != hipSuccess || cur != p->device) {
        na_set_error("plan lives on device %d, current device is %d", p->device, cur);
        return NA_ERR_PLAN_MISMATCH;
    }
    const bool passes = (flags & NA_FWD_PERMUTE_PASSES) && !p->identity_order;
    const size_t need = na_forward_workspace_bytes(p, B, H, flags);
    if (need > 0 && (!workspace || ws_bytes < need || ((uintptr_t)workspace) % 256 != 0)) {
        na_set_error("forward flags 0x%x need %zu bytes of 256-byte aligned workspace", flags,
                     need);
        return NA_ERR_INVALID_ARG;
    }
    // split tail: the r query tiles of the last, partly filled round each run
    // as s workgroups over shares of their walk; s minimises the time of the
    // shares, ceil(r s / capacity) rounds of 1/s of a tile each (the smallest
    // such s), and the split is taken only when that is at most half the one
    // round of whole tiles: each share pays its own Q load, pipeline fill and
    // partial store, so a 1-D causal tail of 3/4 of a round split four ways
    // measured 2% slower than unsplit
    int64_t n_main = n_wg, n_split = 1;
    if (split_ws_bytes(p, flags) > 0) {
        const int64_t cap = p->split_capacity, r = n_wg % cap;
        const int64_t s_max = std::min<int64_t>(kMaxShares, p->max_row_len);
        double best = 0.5 + 1e-9;
        for (int64_t s = 2; r > 0 && s <= s_max && r * s <= kShareRounds * cap; ++s) {
            const double t = (double)((r * s + cap - 1) / cap) / (double)s;
            if (t < best - 1e-9) {
                best = t;
                n_split = s;
            }
        }
        if (n_split > 1) n_main = n_wg - r;
    }

    if (log_level() >= 2)
        std::fprintf(stderr,
                     "na: forward B=%lld H=%lld q_block=%d workgroups=%lld whole=%lld shares=%lld "
                     "(split %lld) flags=0x%x\n",
                     (long long)B, (long long)H, p->desc.q_block, (long long)n_wg, (long long)n_main,
                     (long long)((n_wg - n_main) * n_split), (long long)n_split, flags);
    NaAttnParams a{};
    a.n_tokens = (int32_t)p->n_tokens;
    a.heads = (int32_t)H;
    a.n_q_tiles = (int32_t)p->stats.n_q_tiles;
    a.n_wg = (int32_t)n_wg;
    a.n_main = (int32_t)n_main;
    a.n_split = (int32_t)n_split;
    a.q_desc = p->q_desc ? 1 : 0;
    if (n_split > 1) {
        char* sw = (char*)workspace + permute_ws_bytes(p, B, H, flags);
        const size_t rows = (size_t)(kShareRounds * p->split_capacity) * (size_t)d.q_block;
        a.part_o = (float*)sw;
        a.part_ml = (float*)(sw + up256(rows * (size_t)d.head_dim * sizeof(float)));
    }
    a.scale_log2 = scale * 1.4426950408889634f;
    a.row_ptr = p->d_row_ptr;
    a.entries = p->d_entries;
    a.masks = p->d_masks;
    a.zero = p->d_zero;
    a.lse = lse;
    if (fusion) {
        // delta = z + log(alpha) on window keys, z + log(1 - alpha) on partners:
        // the kernel adds log((1 - alpha) / alpha) to the partners' logits (as a
        // raw dot-product offset) and log(alpha) to lse
        const double alpha = d.skip_prior;
        a.skip_masks = p->d_skip_masks;
        a.skip_bias = (float)(std::log((1.0 - alpha) / alpha) / (double)scale);
        a.lse_shift = (float)std::log(alpha);
    }
    const int64_t N = p->n_tokens, D = d.head_dim, eb = elem_bytes(p);
    // the bf16 kernels with 32 queries per wave take the separate softmax's
    // partner branch in their epilogue; the others (fp32, and the 48-query
    // bf16 kernels at q_block 192 and 384) run it as a second kernel
    const bool sep_fused = separate && d.dtype == NA_BF16 && d.q_block != 192 && d.q_block != 384;
    if (sep_fused) {
        a.sep_skip = d.skip;
        a.sep_both = d.skip_both;
    }

    if (n_wg == 0) return NA_OK;
    int rc = 0;
    if (!passes) {
        a.q = q->ptr;
        a.k = k->ptr;
        a.v = v->ptr;
        a.out = out->ptr;
        a.q_sb = q->stride_b, a.q_sh = q->stride_h, a.q_sn = q->stride_n;
        a.k_sb = k->stride_b, a.k_sh = k->stride_h, a.k_sn = k->stride_n;
        a.v_sb = v->stride_b, a.v_sh = v->stride_h, a.v_sn = v->stride_n;
        a.o_sb = out->stride_b, a.o_sh = out->stride_h, a.o_sn = out->stride_n;
        a.perm = p->identity_order ? nullptr : p->d_perm;
        rc = na_attn_launch(a, d.dtype, d.head_dim, d.q_block, fusion, stream);
    } else {
        // gather q, k, v into sequence order, attend on contiguous tiles, scatter back
        auto up = up256;
        const size_t t = (size_t)(B * H * N * D * eb);
        char* ws = (char*)workspace;
        void* qs = ws;
        void* ks = ws + up(t);
        void* vs = ws + 2 * up(t);
        void* os = ws + 3 * up(t);
        float* ls = (float*)(ws + 4 * up(t));
        const int64_t csb = H * N * D * eb, csh = N * D * eb, csn = D * eb;
        const na_tensor* src[3] = {q, k, v};
        void* dst[3] = {qs, ks, vs};
        for (int i = 0; i < 3 && rc == 0; ++i)
            rc = na_permute_launch(src[i]->ptr, dst[i], B, H, N, D * eb, src[i]->stride_b * eb,
                                   src[i]->stride_h * eb, src[i]->stride_n * eb, csb, csh, csn,
                                   p->d_perm, 0, stream);
        if (rc == 0) {
            a.q = qs, a.k = ks, a.v = vs, a.out = os;
            a.q_sb = a.k_sb = a.v_sb = a.o_sb = H * N * D;
            a.q_sh = a.k_sh = a.v_sh = a.o_sh = N * D;
            a.q_sn = a.k_sn = a.v_sn = a.o_sn = D;
            a.perm = nullptr;
            a.lse = lse ? ls : nullptr;
            rc = na_attn_launch(a, d.dtype, d.head_dim, d.q_block, fusion, stream);
        }
        if (rc == 0)
            rc = na_permute_launch(os, out->ptr, B, H, N, D * eb, csb, csh, csn,
                                   out->stride_b * eb, out->stride_h * eb, out->stride_n * eb,
                                   p->d_perm, 1, stream);
        if (rc == 0 && lse)
            rc = na_permute_launch(ls, lse, B, H, N, 4, H * N * 4, N * 4, 4, H * N * 4, N * 4, 4,
                                   p->d_perm, 1, stream);
    }
    if (rc == 0 && separate && !sep_fused) {
        // the partner branch of the separate-softmax variant, added to out
        NaSkipParams sp{};
        sp.q = q->ptr, sp.k = k->ptr, sp.v = v->ptr, sp.out = out->ptr;
        sp.q_sb = q->stride_b, sp.q_sh = q->stride_h, sp.q_sn = q->stride_n;
        sp.k_sb = k->stride_b, sp.k_sh = k->stride_h, sp.k_sn = k->stride_n;
        sp.v_sb = v->stride_b, sp.v_sh = v->stride_h, sp.v_sn = v->stride_n;
        sp.o_sb = out->stride_b, sp.o_sh = out->stride_h, sp.o_sn = out->stride_n;
        sp.batch = (int32_t)B, sp.heads = (int32_t)H, sp.n_tokens = (int32_t)N;
        sp.skip = d.skip, sp.skip_both = d.skip_both, sp.scale = scale;
        sp.perm = p->identity_order ? nullptr : p->d_perm;
        rc = na_skip_launch(sp, d.dtype, d.head_dim, stream);
    }
    if (rc != 0) {
        na_set_error("kernel launch failed: %s", hip_err((hipError_t)rc));
        return NA_ERR_DEVICE;
    }
    return NA_OK;
}

size_t na_backward_workspace_bytes(na_plan_t p, int64_t B, int64_t H) {
    if (!p || B < 1 || H < 1) return 0;
    return ((size_t)B * (size_t)H * (size_t)p->n_tokens * sizeof(float) + 255) & ~(size_t)255;
}

na_status na_backward(na_plan_t p, int64_t B, int64_t H, const na_tensor* q, const na_tensor* k,
                      const na_tensor* v, const na_tensor* out, const na_tensor* dout,
                      const float* lse, const na_tensor* dq, const na_tensor* dk,
                      const na_tensor* dv, float scale, void* workspace, size_t ws_bytes,
                      void* stream) {
    if (!p) {
        na_set_error("plan is NULL");
        return NA_ERR_INVALID_ARG;
    }
    if (!p->on_device) {
        na_set_error("plan was built host-only and cannot run");
        return NA_ERR_PLAN_MISMATCH;
    }
    if (B < 1 || H < 1) {
        na_set_error("B and H must be >= 1");
        return NA_ERR_INVALID_ARG;
    }
    const int64_t nq = p->stats.n_q_tiles * B * H, nk = p->stats.n_kv_tiles * B * H;
    if (nq > 0x7fffffff || nk > 0x7fffffff || B * H > 0x7fffffff / (p->n_tokens > 0 ? p->n_tokens : 1)) {
        na_set_error("B * H * tiles too large");
        return NA_ERR_INVALID_ARG;
    }
    na_status st;
    const na_tensor* ts[8] = {q, k, v, out, dout, dq, dk, dv};
    const char* names[8] = {"q", "k", "v", "out", "dout", "dq", "dk", "dv"};
    for (int i = 0; i < 8; ++i)
        if ((st = check_tensor(p, ts[i], names[i], B, H)) != NA_OK) return st;
    if (!lse || ((uintptr_t)lse) % 4 != 0) {
        na_set_error("lse must be a 4-byte aligned fp32 [B, H, N] array");
        return NA_ERR_INVALID_ARG;
    }
    if (!(scale > 0.f) || scale == __builtin_inff()) {
        na_set_error("scale must be finite and positive");
        return NA_ERR_INVALID_ARG;
    }
    const na_plan_desc& d = p->desc;
    const bool fusion = d.skip > 0 && d.skip_mode == NA_SKIP_FIXED_FUSION;
    const bool separate = d.skip > 0 && d.skip_mode == NA_SKIP_SEPARATE;
    if (!na_bwd_supported(d.dtype, d.head_dim, d.q_block, d.kv_block)) {
        na_set_error("no gradient kernels for dtype=%d head_dim=%d q_block=%d kv_block=%d",
                     d.dtype, d.head_dim, d.q_block, d.kv_block);
        return NA_ERR_UNSUPPORTED;
    }
    const size_t need = na_backward_workspace_bytes(p, B, H);
    if (!workspace || ws_bytes < need || ((uintptr_t)workspace) % 256 != 0) {
        na_set_error("backward needs %zu bytes of 256-byte aligned workspace", need);
        return NA_ERR_INVALID_ARG;
    }
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != p->device) {
        na_set_error("plan lives on device %d, current device is %d", p->device, cur);
        return NA_ERR_PLAN_MISMATCH;
    }
    NaBwdParams a{};
    a.q = q->ptr, a.k = k->ptr, a.v = v->ptr, a.out = out->ptr, a.dout = dout->ptr;
    a.dq = dq->ptr, a.dk = dk->ptr, a.dv = dv->ptr;
    a.lse = lse;
    a.delta = (float*)workspace;
    a.q_sb = q->stride_b, a.q_sh = q->stride_h, a.q_sn = q->stride_n;
    a.k_sb = k->stride_b, a.k_sh = k->stride_h, a.k_sn = k->stride_n;
    a.v_sb = v->stride_b, a.v_sh = v->stride_h, a.v_sn = v->stride_n;
    a.o_sb = out->stride_b, a.o_sh = out->stride_h, a.o_sn = out->stride_n;
    a.g_sb = dout->stride_b, a.g_sh = dout->stride_h, a.g_sn = dout->stride_n;
    a.dq_sb = dq->stride_b, a.dq_sh = dq->stride_h, a.dq_sn = dq->stride_n;
    a.dk_sb = dk->stride_b, a.dk_sh = dk->stride_h, a.dk_sn = dk->stride_n;
    a.dv_sb = dv->stride_b, a.dv_sh = dv->stride_h, a.dv_sn = dv->stride_n;
    a.batch = (int32_t)B;
    a.n_tokens = (int32_t)p->n_tokens;
    a.heads = (int32_t)H;
    a.n_q_tiles = (int32_t)p->stats.n_q_tiles;
    a.n_kv_tiles = (int32_t)p->stats.n_kv_tiles;
    a.q_block = (int32_t)d.q_block;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.perm = p->identity_order ? nullptr : p->d_perm;
    a.row_ptr = p->d_row_ptr;
    a.entries = p->d_entries;
    a.t_row_ptr = p->d_t_row_ptr;
    a.t_entries = p->d_t_entries;
    a.p_row_ptr = p->d_p_row_ptr;
    a.p_entries = p->d_p_entries;
    a.masks = p->d_masks;
    a.zero = p->d_zero;
    if (fusion) {  // the forward's logit bias and lse shift (see na_forward)
        const double alpha = d.skip_prior;
        a.skip_masks = p->d_skip_masks;
        a.skip_bias = (float)(std::log((1.0 - alpha) / alpha) / (double)scale);
        a.lse_shift = (float)std::log(alpha);
    }
    a.skip = d.skip;
    a.skip_both = d.skip_both;
    if (p->n_tokens == 0) return NA_OK;
    int rc = 0;
    if (separate) {
        // the window branch over the plan's (window-only) map with the window
        // branch's own row sums, then the partner branch's gradients added
        rc = na_skip_bwd_delta_launch(a, d.head_dim, stream);
        if (rc == 0) rc = na_bwd_launch(a, d.head_dim, false, false, stream);
        if (rc == 0) rc = na_skip_bwd_grads_launch(a, d.head_dim, stream);
    } else {
        rc = na_bwd_launch(a, d.head_dim, fusion, true, stream);
    }
    if (rc != 0) {
        na_set_error("kernel launch failed: %s", hip_err((hipError_t)rc));
        return NA_ERR_DEVICE;
    }
    return NA_OK;
}

na_status na_backward_noalloc(na_plan_t p, int64_t B, int64_t H, const na_tensor* q,
                              const na_tensor* k, const na_tensor* v, const na_tensor* out,
                              const na_tensor* dout, const float* lse, const na_tensor* dq,
                              const na_tensor* dk, const na_tensor* dv, float scale,
                              void* stream) {
    if (!p) {
        na_set_error("plan is NULL");
        return NA_ERR_INVALID_ARG;
    }
    if (B < 1 || H < 1) {
        na_set_error("B and H must be >= 1");
        return NA_ERR_INVALID_ARG;
    }
    // (in double: no overflow; the limit is a multiple of 256, so this is
    // na_backward_workspace_bytes(p, B, H) <= the limit)
    if ((double)B * (double)H * (double)p->n_tokens * sizeof(float) >
        (double)NA_BACKWARD_NOALLOC_MAX_BYTES) {
        na_set_error("na_backward_noalloc: B * H * N = %lld * %lld * %lld delta rows exceed the "
                     "fixed scratch of %u bytes (%u rows); use na_backward with a workspace",
                     (long long)B, (long long)H, (long long)p->n_tokens,
                     (unsigned)NA_BACKWARD_NOALLOC_MAX_BYTES,
                     (unsigned)(NA_BACKWARD_NOALLOC_MAX_BYTES / sizeof(float)));
        return NA_ERR_INVALID_ARG;
    }
    if (!p->on_device) {
        na_set_error("plan was built host-only and cannot run");
        return NA_ERR_PLAN_MISMATCH;
    }
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != p->device) {
        na_set_error("plan lives on device %d, current device is %d", p->device, cur);
        return NA_ERR_PLAN_MISMATCH;
    }
    void* ws = nullptr;
    size_t ws_bytes = 0;
    const int rc = na_bwd_scratch(&ws, &ws_bytes);
    if (rc != 0) {
        na_set_error("device scratch lookup failed: %s", hip_err((hipError_t)rc));
        return NA_ERR_DEVICE;
    }
    return na_backward(p, B, H, q, k, v, out, dout, lse, dq, dk, dv, scale, ws, ws_bytes, stream);
}

na_status na_permute(na_plan_t p, int64_t B, int64_t H, const na_tensor* in, const na_tensor* out,
                     int32_t inverse, void* stream) {
    if (!p) {
        na_set_error("plan is NULL");
        return NA_ERR_INVALID_ARG;
    }
    if (!p->on_device) {
        na_set_error("plan was built host-only and cannot run");
        return NA_ERR_PLAN_MISMATCH;
    }
    if (B < 1 || H < 1 || (inverse != 0 && inverse != 1)) {
        na_set_error("B, H must be >= 1 and inverse 0 or 1");
        return NA_ERR_INVALID_ARG;
    }
    na_status st;
    if ((st = check_tensor(p, in, "in", B, H)) != NA_OK) return st;
    if ((st = check_tensor(p, out, "out", B, H)) != NA_OK) return st;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess || cur != p->device) {
        na_set_error("plan lives on device %d, current device is %d", p->device, cur);
        return NA_ERR_PLAN_MISMATCH;
    }
    if (p->identity_order) {
        na_set_error("the plan's order is the identity: nothing to permute");
        return NA_ERR_UNSUPPORTED;
    }
    const int64_t eb = elem_bytes(p);
    int rc;
    rc = na_permute_launch(in->ptr, out->ptr, B, H, p->n_tokens, p->desc.head_dim * eb,
                           in->stride_b * eb, in->stride_h * eb, in->stride_n * eb,
                           out->stride_b * eb, out->stride_h * eb, out->stride_n * eb, p->d_perm,
                           inverse, stream);
    if (rc != 0) {
        na_set_error("permute launch failed: %s", hip_err((hipError_t)rc));
        return NA_ERR_DEVICE;
    }
    return NA_OK;
}

}  // extern "C"
