// C ABI of the Occult MoE-layer library: argument checks, workspace layout,
// and the stage sequence of the layer (declarations and contracts in occ.h).
#include <algorithm>
#include <mutex>
#include <vector>

#include "launch.h"

#pragma GCC visibility push(default)
#include "occ.h"
#pragma GCC visibility pop

using namespace occ;

namespace occ {
int compute_units() {
    constexpr int kDevices = 64;
    static int cached[kDevices] = {};  // 0: not read yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 256;
    int v = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        __atomic_store_n(&cached[dev], v, __ATOMIC_RELAXED);
    }
    return v;
}
}  // namespace occ

// The allocation-free forward's workspace: a file-scope device array that
// each GPU holds (at its own address) from the library's load until the
// process ends.  In host code `scratch` is only a stand-in for the symbol;
// its device address on the current GPU is looked up once per device with
// hipGetSymbolAddress (noalloc_scratch below) and that address is what
// kernels receive.  Every call on one GPU uses the same array, so calls that
// overlap on a GPU race.
static __device__ __align__(256) unsigned char scratch[OCC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

size_t elem_bytes(const occ_layer_desc &D) { return D.dtype == OCC_BF16 ? 2 : 4; }
// The grouped GEMM kernels for a shape.  bf16 batches whose experts average
// fewer than kSmallTileRows rows (T*k < 96*Ne, e.g. decode steps) take the
// 128-row tiles, whose smaller LDS slices leave room for a third ring slot:
// such launches stream the weights from HBM.  The choice is made from the
// shape alone (nothing is read back): an average of 96 keeps the largest
// expert within one 128-row tile at the spread of expert loads seen in
// routed batches (the largest about 1.25x the average), and above it an
// expert's second 128-row tile costs a round of the CUs that one 320-row
// tile avoids (OLMoE shape: 128-row tiles 7% faster at 700 tokens, 5%
// slower at 1000).
struct GemmOps {
    hipError_t (*up)(const UpArgs &, size_t, hipStream_t);
    hipError_t (*down)(const DownArgs &, size_t, hipStream_t);
    int bm;
};
GemmOps gemm_ops(const occ_layer_desc &D) {
    if (D.dtype != OCC_BF16) return {launch_gemm_up_f32, launch_gemm_down_f32, kGemmBmF32};
    if (static_cast<int64_t>(D.T) * D.k < static_cast<int64_t>(kSmallTileRows) * D.Ne)
        return {launch_gemm_up_bf16_m128, launch_gemm_down_bf16_m128, kGemmBmBf16Small};
    return {launch_gemm_up_bf16, launch_gemm_down_bf16, kGemmBmBf16};
}
int tile_rows(const occ_layer_desc &D) { return gemm_ops(D).bm; }
// The routed row-tile schedule fills the up-projection's last round of the
// CUs on the 320-row build (column tiles of 128 features); the other builds
// take ceil(rows / capacity) tiles per expert.
int fill_cols(const occ_layer_desc &D) {
    return gemm_ops(D).up == launch_gemm_up_bf16 ? static_cast<int>(ceil_div(D.F, 128)) : 0;
}

// Dense products (the shared experts) that fill at least kDensePipeRounds
// rounds of the CUs with 256 x 256 tiles take the pipelined four-wave build;
// cols is the product's MFMA output width (the up-projection's gate and up
// columns together).
bool dense_pipelined(const GemmOps &ops, int64_t M, int64_t cols) {
    if (ops.up != launch_gemm_up_bf16) return false;  // fp32, or the decode regime
    const int64_t tiles = ((M + 255) / 256) * ((cols + 255) / 256);
    return tiles >= static_cast<int64_t>(kDensePipeRounds) * compute_units();
}

// Byte offsets of every buffer inside the workspace.  Sized for the worst
// case N_sfd = T * min(k, Nd), so no data-dependent size is read back.
struct Layout {
    size_t logits, ids, w, brim0, sfd_off, epd_off, tile_off, tile_off_first, tile_off_rest, first_cnt,
        chunk_cnt, chunk_base, epd_src, epd_w, tok_epd, down_rows, brim1, brim_end, x_sfd, epd,
        sfd_out, h_sh, y_sh, y_epd;
    // training only (flags & OCC_FLAG_TRAIN): saved pre-activations and the
    // backward pass's buffers
    size_t gu, gu_sh, dy_sfd, dgu, dx_sfd, dw_part, zero_row, bt_all, bt_first, bt_rest, dgu_sh,
        dx_sh, wt_sh, wt_down, dense_seg, dense_tile, wg_part;
    int dw_stride;
    size_t total;
};

constexpr int kBwdTile = 256;  // rows and columns of a backward GEMM tile

Layout layout(const occ_layer_desc &D) {
    const size_t T = D.T, k = D.k, Nd = D.Nd, Ne = D.Ne, d = D.d, F = D.F, es = elem_bytes(D);
    const size_t n = Ne / Nd, nsfd_max = T * std::min(k, Nd), nepd = T * k;
    const size_t nchunks = (T + kBrimChunk - 1) / kBrimChunk, nb = Nd + 2 * Ne;
    Layout L{};
    size_t o = 0;
    auto take = [&o](size_t bytes) {
        const size_t r = o;
        o = align_up(o + std::max<size_t>(bytes, 1));
        return r;
    };
    L.logits = take(T * Ne * 4);
    L.ids = take(nepd * 4);
    L.w = take(nepd * 4);
    L.brim0 = take(Nd * T * 4);
    L.sfd_off = take((Nd + 1) * 4);
    L.epd_off = take((Ne + 1) * 4);
    L.tile_off = take((Ne + 1) * 4);
    L.tile_off_first = take((Ne + 1) * 4);
    L.tile_off_rest = take((Ne + 1) * 4);
    L.first_cnt = take(Ne * 4);
    L.chunk_cnt = take(nchunks * nb * 4);
    L.chunk_base = take(nchunks * nb * 4);
    L.epd_src = take(nepd * 4);
    L.epd_w = take(nepd * 4);
    L.tok_epd = take(nepd * 4);
    L.down_rows = take(nepd * 4);
    L.brim1 = take(n * nsfd_max * 4);
    L.brim_end = o;
    L.x_sfd = take(nsfd_max * d * es);
    L.epd = take(nepd * F * es);
    L.sfd_out = take(nsfd_max * d * 4);
    // deterministic merge: every EPD row's fp32 result (the backward reuses
    // it for dx)
    if (D.flags & OCC_FLAG_DETERMINISTIC) L.y_epd = take(nepd * d * 4);
    const size_t Nsh = static_cast<size_t>(D.n_shared) * D.F_shared;
    if (D.n_shared > 0) {
        L.h_sh = take(T * Nsh * es);
        L.y_sh = take(T * d * 4);
    }
    if (D.flags & OCC_FLAG_TRAIN) {
        L.dw_stride = 2 * static_cast<int>((F + kBwdTile - 1) / kBwdTile);
        L.gu = take(nepd * 2 * F * es);
        L.dy_sfd = take(nsfd_max * d * es);
        L.dgu = take(nepd * 2 * F * es);
        L.dx_sfd = take(nsfd_max * d * 4);
        L.dw_part = take(nepd * L.dw_stride * 4);
        L.zero_row = take(std::max<size_t>({d, 2 * F, 2 * Nsh, kBwdTile}) * es);
        L.bt_all = take((Ne + 1) * 4);
        L.bt_first = take((Ne + 1) * 4);
        L.bt_rest = take((Ne + 1) * 4);
        L.dense_seg = take(2 * 4);
        L.dense_tile = take(2 * 4);
        if (D.n_shared > 0) {
            L.gu_sh = take(T * 2 * Nsh * es);
            L.dgu_sh = take(T * 2 * Nsh * es);
            L.dx_sh = take(T * d * 4);
            // the shared gate and up weights transposed, d x 2 F_shared per
            // expert (the input gradient's contraction index contiguous)
            L.wt_sh = take(Nsh * d * 2 * es);
            // and the shared down-projection weights, F_shared x d per
            // expert, for dh_sh = dy W_d read K-contiguous
            L.wt_down = take(Nsh * d * es);
            // the shared weight gradients' split-K partials (dense, K = T)
            const size_t Fs = D.F_shared, nsh = D.n_shared;
            const size_t p3 = wgrad_k_parts(D.n_shared, D.d, D.F_shared, D.T);
            const size_t p4 = wgrad_k_parts(D.n_shared, 2 * D.F_shared, D.d, D.T);
            const size_t need = std::max(p3 > 1 ? p3 * nsh * d * Fs : 0,
                                         p4 > 1 ? p4 * nsh * 2 * Fs * d : 0);
            L.wg_part = need ? take(need * 4) : 0;
        }
    }
    L.total = o;
    return L;
}

occ_status check_desc(const occ_layer_desc *D) {
    if (!D) return OCC_ERR_INVALID_ARG;
    if (D->T < 1 || D->d < 1 || D->Ne < 1 || D->k < 1 || D->Nd < 1 || D->F < 1)
        return OCC_ERR_INVALID_ARG;
    if (D->k > D->Ne || D->Ne % D->Nd != 0) return OCC_ERR_INVALID_ARG;
    if (D->n_shared < 0 || (D->n_shared > 0 && D->F_shared < 1)) return OCC_ERR_INVALID_ARG;
    if (D->dtype != OCC_F32 && D->dtype != OCC_BF16) return OCC_ERR_INVALID_ARG;
    if (D->prune_rule < OCC_PRUNE_OFF || D->prune_rule > OCC_PRUNE_SIMILARITY)
        return OCC_ERR_INVALID_ARG;
    if (D->prune_rule != OCC_PRUNE_OFF &&
        (D->prune_groups < 1 ||
         static_cast<int64_t>(D->prune_groups) * (D->Ne / D->Nd) < D->k))
        return OCC_ERR_INVALID_ARG;
    if (D->flags & ~(OCC_FLAG_TRAIN | OCC_FLAG_DETERMINISTIC)) return OCC_ERR_INVALID_ARG;
    // training keeps bf16 pre-activations for the bf16 backward GEMMs, whose
    // 256-wide tiles need d, F (and F_shared) of at least 256
    if ((D->flags & OCC_FLAG_TRAIN) &&
        (D->dtype != OCC_BF16 || D->d < kBwdTile || D->F < kBwdTile ||
         (D->n_shared > 0 && D->F_shared < kBwdTile)))
        return OCC_ERR_UNSUPPORTED;
    if (D->Ne > kMaxNe || D->Nd > kMaxNd || D->k > kMaxK) return OCC_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(D->T) * D->k >= (1ll << 31) ||
        static_cast<int64_t>(D->T) * D->Nd >= (1ll << 31))
        return OCC_ERR_UNSUPPORTED;
    const int mult = D->dtype == OCC_BF16 ? 64 : 16;
    if (D->d % mult || D->F % mult || (D->n_shared > 0 && D->F_shared % mult))
        return OCC_ERR_UNSUPPORTED;
    if (D->d > (D->dtype == OCC_BF16 ? 8192 : 4096)) return OCC_ERR_UNSUPPORTED;
    return OCC_OK;
}

occ_status make_tab(const occ_layer_desc &D, const int32_t *L, PlaceTab *tab) {
    if (!L) return OCC_ERR_INVALID_ARG;
    const int n = D.Ne / D.Nd;
    bool seen[kMaxNe] = {};
    *tab = PlaceTab{};
    for (int g = 0; g < D.Nd; g++)
        for (int j = 0; j < n; j++) {
            const int e = L[g * n + j];
            if (e < 0 || e >= D.Ne || seen[e]) return OCC_ERR_INVALID_ARG;
            seen[e] = true;
            tab->grp[e] = static_cast<uint8_t>(g);
            tab->slot[e] = static_cast<uint8_t>(j);
            tab->expert[g * n + j] = static_cast<uint8_t>(e);
        }
    tab->Ne = D.Ne;
    tab->Nd = D.Nd;
    tab->n = n;
    return OCC_OK;
}

occ_status check_ws(const occ_layer_desc &D, const void *ws, size_t ws_bytes, size_t need) {
    (void)D;
    if (!ws || reinterpret_cast<uintptr_t>(ws) % kAlign != 0 || ws_bytes < need)
        return OCC_ERR_WORKSPACE;
    return OCC_OK;
}

template <typename T>
T *at(void *ws, size_t off) {
    return reinterpret_cast<T *>(static_cast<char *>(ws) + off);
}

occ_brim brim_view(void *ws, const Layout &L) {
    occ_brim b;
    b.brim0 = at<int32_t>(ws, L.brim0);
    b.sfd_off = at<int32_t>(ws, L.sfd_off);
    b.epd_off = at<int32_t>(ws, L.epd_off);
    b.epd_src = at<int32_t>(ws, L.epd_src);
    b.epd_w = at<float>(ws, L.epd_w);
    b.tok_epd = at<int32_t>(ws, L.tok_epd);
    b.brim1 = at<int32_t>(ws, L.brim1);
    b.down_rows = at<int32_t>(ws, L.down_rows);
    b.first_cnt = at<int32_t>(ws, L.first_cnt);
    b.tile_off = at<int32_t>(ws, L.tile_off);
    return b;
}

BrimBufs brim_bufs(void *ws, const Layout &L) {
    BrimBufs b;
    b.brim0 = at<int32_t>(ws, L.brim0);
    b.sfd_off = at<int32_t>(ws, L.sfd_off);
    b.epd_off = at<int32_t>(ws, L.epd_off);
    b.tile_off = at<int32_t>(ws, L.tile_off);
    b.epd_src = at<int32_t>(ws, L.epd_src);
    b.tok_epd = at<int32_t>(ws, L.tok_epd);
    b.brim1 = at<int32_t>(ws, L.brim1);
    b.epd_w = at<float>(ws, L.epd_w);
    b.down_rows = at<int32_t>(ws, L.down_rows);
    b.first_cnt = at<int32_t>(ws, L.first_cnt);
    b.tile_off_first = at<int32_t>(ws, L.tile_off_first);
    b.tile_off_rest = at<int32_t>(ws, L.tile_off_rest);
    b.chunk_cnt = at<int32_t>(ws, L.chunk_cnt);
    b.chunk_base = at<int32_t>(ws, L.chunk_base);
    return b;
}

occ_status hip_status(hipError_t e) { return e == hipSuccess ? OCC_OK : OCC_ERR_HIP; }

// Row tiles of a dense backward input-gradient product over T rows against
// n_tiles column tiles: ceil(T / kBwdRowTile), raised as far as the launch
// keeps the same number of rounds of the CUs (one workgroup each), so the
// last round is filled with shorter tiles; at most one 16-row block per tile.
int dense_row_tiles_bwd(int T, int n_tiles) {
    const long m0 = (T + kBwdRowTile - 1) / kBwdRowTile, cus = compute_units();
    if (m0 == 0 || n_tiles <= 0) return static_cast<int>(m0);
    const long rounds = (m0 * n_tiles + cus - 1) / cus;
    const long m = std::min<long>(rounds * cus / n_tiles, (T + 15) / 16);
    return static_cast<int>(std::max(m0, m));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

occ_status noalloc_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return OCC_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return OCC_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return OCC_ERR_HIP;
        if (reinterpret_cast<uintptr_t>(p) % kAlign != 0) return OCC_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return OCC_OK;
}

#define OCC_TRY(expr)                              \
    do {                                           \
        const occ_status st_ = (expr);             \
        if (st_ != OCC_OK) return st_;             \
    } while (0)

#define OCC_HIP(expr) OCC_TRY(hip_status(expr))

}  // namespace

extern "C" {

const char *occ_status_string(occ_status s) {
    switch (s) {
        case OCC_OK: return "OCC_OK";
        case OCC_ERR_INVALID_ARG: return "OCC_ERR_INVALID_ARG";
        case OCC_ERR_UNSUPPORTED: return "OCC_ERR_UNSUPPORTED";
        case OCC_ERR_WORKSPACE: return "OCC_ERR_WORKSPACE";
        case OCC_ERR_HIP: return "OCC_ERR_HIP";
    }
    return "OCC_ERR_UNKNOWN";
}

occ_status occ_workspace_size(const occ_layer_desc *desc, size_t *bytes_host) {
    OCC_TRY(check_desc(desc));
    if (!bytes_host) return OCC_ERR_INVALID_ARG;
    *bytes_host = layout(*desc).total;
    return OCC_OK;
}

occ_status occ_route(const occ_layer_desc *desc, const float *logits,
                     const int32_t *placement_host, int32_t *ids, float *w, void *stream) {
    OCC_TRY(check_desc(desc));
    if (!logits || !ids || !w || desc->prune_rule == OCC_PRUNE_SIMILARITY)
        return OCC_ERR_INVALID_ARG;
    PlaceTab tab;
    OCC_TRY(make_tab(*desc, placement_host, &tab));
    OCC_HIP(launch_route(logits, desc->T, desc->Ne, desc->k, desc->prune_rule,
                         desc->prune_groups, tab, nullptr, ids, w,
                         static_cast<hipStream_t>(stream)));
    return OCC_OK;
}

occ_status occ_similarity_accumulate(int32_t T, int32_t Ne, const float *logits, double *gram,
                                     void *stream) {
    if (T < 0 || Ne < 1 || Ne > kMaxNe || !gram || (T > 0 && !logits)) return OCC_ERR_INVALID_ARG;
    OCC_HIP(launch_sim_gram(logits, T, Ne, gram, static_cast<hipStream_t>(stream)));
    return OCC_OK;
}

occ_status occ_similarity_rank(int32_t Ne, const double *gram, double *t2, int32_t *rank,
                               void *stream) {
    if (Ne < 1 || Ne > kMaxNe || !gram || !rank) return OCC_ERR_INVALID_ARG;
    OCC_HIP(launch_sim_rank(gram, Ne, t2, rank, static_cast<hipStream_t>(stream)));
    return OCC_OK;
}

occ_status occ_route_similarity(const occ_layer_desc *desc, const float *logits,
                                const int32_t *placement_host, const int32_t *sim_rank,
                                int32_t *ids, float *w, void *stream) {
    OCC_TRY(check_desc(desc));
    if (!logits || !ids || !w || !sim_rank || desc->prune_rule != OCC_PRUNE_SIMILARITY)
        return OCC_ERR_INVALID_ARG;
    PlaceTab tab;
    OCC_TRY(make_tab(*desc, placement_host, &tab));
    OCC_HIP(launch_route(logits, desc->T, desc->Ne, desc->k, desc->prune_rule,
                         desc->prune_groups, tab, sim_rank, ids, w,
                         static_cast<hipStream_t>(stream)));
    return OCC_OK;
}

occ_status occ_build_brim(const occ_layer_desc *desc, const int32_t *ids, const float *w,
                          const int32_t *placement_host, int dense_brim1, void *workspace,
                          size_t ws_bytes, occ_brim *out_host, void *stream) {
    OCC_TRY(check_desc(desc));
    if (!ids || !w || !out_host) return OCC_ERR_INVALID_ARG;
    PlaceTab tab;
    OCC_TRY(make_tab(*desc, placement_host, &tab));
    const Layout L = layout(*desc);
    OCC_TRY(check_ws(*desc, workspace, ws_bytes, L.brim_end));
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t *ids_ws = at<int32_t>(workspace, L.ids);
    float *w_ws = at<float>(workspace, L.w);
    OCC_HIP(launch_sanitize_ids(ids, w, desc->T, desc->k, desc->Ne, ids_ws, w_ws, s));
    OCC_HIP(launch_brim(ids_ws, w_ws, desc->T, desc->k, tab, tile_rows(*desc), fill_cols(*desc),
                        dense_brim1 != 0, brim_bufs(workspace, L), s));
    *out_host = brim_view(workspace, L);
    return OCC_OK;
}

occ_status occ_forward_views(const occ_layer_desc *desc, void *workspace,
                             occ_forward_view *out_host) {
    OCC_TRY(check_desc(desc));
    if (!workspace || !out_host) return OCC_ERR_INVALID_ARG;
    const Layout L = layout(*desc);
    occ_forward_view v;
    v.logits = at<float>(workspace, L.logits);
    v.ids = at<int32_t>(workspace, L.ids);
    v.w = at<float>(workspace, L.w);
    v.brim = brim_view(workspace, L);
    v.x_sfd = at<void>(workspace, L.x_sfd);
    v.epd = at<void>(workspace, L.epd);
    v.sfd_out = at<float>(workspace, L.sfd_out);
    v.h_shared = desc->n_shared > 0 ? at<void>(workspace, L.h_sh) : nullptr;
    v.y_shared = desc->n_shared > 0 ? at<float>(workspace, L.y_sh) : nullptr;
    *out_host = v;
    return OCC_OK;
}

// The layer's stage sequence.  Stage 0 routes `logits` (the desc's rule),
// or first computes them as x w_router^T when w_router is given, or, with
// neither, copies the caller's routing ids_in / w_in.
static occ_status forward(const occ_layer_desc *desc, const void *x, const float *logits,
                          const void *w_router, const int32_t *ids_in, const float *w_in,
                          const int32_t *placement_host, const void *w_gate, const void *w_up,
                          const void *w_down, const void *ws_gate, const void *ws_up,
                          const void *ws_down, void *y, void *workspace, size_t ws_bytes,
                          void *const *stage_events, void *stream) {
    OCC_TRY(check_desc(desc));
    const occ_layer_desc &D = *desc;
    if (!x || !w_gate || !w_up || !w_down || !y) return OCC_ERR_INVALID_ARG;
    const bool routes = logits || w_router;
    if (routes ? D.prune_rule == OCC_PRUNE_SIMILARITY : (!ids_in || !w_in))
        return OCC_ERR_INVALID_ARG;
    if (D.n_shared > 0 && (!ws_gate || !ws_up || !ws_down)) return OCC_ERR_INVALID_ARG;
    if (stage_events)
        for (int i = 0; i <= OCC_STAGE_COUNT; i++)
            if (!stage_events[i]) return OCC_ERR_INVALID_ARG;
    PlaceTab tab;
    OCC_TRY(make_tab(D, placement_host, &tab));
    const Layout L = layout(D);
    OCC_TRY(check_ws(D, workspace, ws_bytes, L.total));

    hipStream_t s = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) -> occ_status {
        if (!stage_events) return OCC_OK;
        return hip_status(hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s));
    };
    const bool bf16 = D.dtype == OCC_BF16;
    const size_t es = elem_bytes(D);
    const BrimBufs bb = brim_bufs(workspace, L);
    int32_t *ids = at<int32_t>(workspace, L.ids);
    float *w = at<float>(workspace, L.w);
    void *x_sfd = at<void>(workspace, L.x_sfd);
    void *epd = at<void>(workspace, L.epd);
    float *sfd_out = at<float>(workspace, L.sfd_out);
    float *y_sh = D.n_shared > 0 ? at<float>(workspace, L.y_sh) : nullptr;
    const size_t T = D.T;
    const GemmOps ops = gemm_ops(D);
    const size_t bm = ops.bm;
    const size_t routed_tiles = (T * D.k + bm - 1) / bm + D.Ne + kBrimMaxFill;
    const size_t shared_tiles = (T + bm - 1) / bm;

    OCC_TRY(mark(0));
    // Eq. 2: router, behind the gate projection g(x) when its weights are
    // given (or the caller's routing, checked)
    if (w_router) {
        float *lg = at<float>(workspace, L.logits);
        OCC_HIP(launch_gate(x, w_router, D.T, D.d, D.Ne, bf16, lg, s));
        logits = lg;
    }
    if (logits)
        OCC_HIP(launch_route(logits, D.T, D.Ne, D.k, D.prune_rule, D.prune_groups, tab, nullptr,
                             ids, w, s));
    else
        OCC_HIP(launch_sanitize_ids(ids_in, w_in, D.T, D.k, D.Ne, ids, w, s));
    OCC_TRY(mark(1));
    // Algorithms 3 and 5: BRIM_0, BRIM_1 (condensed), GEMM tile schedule
    OCC_HIP(launch_brim(ids, w, D.T, D.k, tab, static_cast<int>(bm), fill_cols(D), 0, bb, s));
    OCC_TRY(mark(2));
    // Small batches (experts averaging fewer than 128 rows) merge in one
    // down-projection launch of atomic adds, whose SFD accumulator rows the
    // dispatch zeroes as it writes the same rows of x_sfd.
    const bool det = D.flags & OCC_FLAG_DETERMINISTIC;
    const bool one_launch = !det && static_cast<int64_t>(D.T) * D.k < 128ll * D.Ne;
    // Algorithm 4: ORI -> SFD
    OCC_HIP(launch_dispatch(x, D.T, D.Nd, static_cast<size_t>(D.d) * es, bb.brim0, x_sfd, s,
                            one_launch ? sfd_out : nullptr, D.d));
    OCC_TRY(mark(3));
    // shared experts: dense SwiGLU over all T tokens, fp32 result
    if (D.n_shared > 0) {
        UpArgs su{};
        su.A = x;
        su.Wg = ws_gate;
        su.Wu = ws_up;
        su.out = at<void>(workspace, L.h_sh);
        su.gu_out = (D.flags & OCC_FLAG_TRAIN) ? at<void>(workspace, L.gu_sh) : nullptr;
        su.M = D.T;
        su.K = D.d;
        su.N = D.n_shared * D.F_shared;
        su.Ne = 1;
        su.tab = tab;
        DownArgs sd{};
        sd.A = su.out;
        sd.W = ws_down;
        sd.out = y_sh;
        sd.M = D.T;
        sd.K = su.N;
        sd.N = D.d;
        sd.Ne = 1;
        sd.k_split = D.F_shared;
        sd.tab = tab;
        if (dense_pipelined(ops, D.T, 2ll * su.N))
            OCC_HIP(launch_gemm_up_bf16_dense(su, shared_tiles, s));
        else
            OCC_HIP(ops.up(su, shared_tiles, s));
        OCC_TRY(mark(4));
        if (dense_pipelined(ops, D.T, sd.N))
            OCC_HIP(launch_gemm_down_bf16_dense(sd, shared_tiles, s));
        else
            OCC_HIP(ops.down(sd, shared_tiles, s));
    } else {
        OCC_TRY(mark(4));
    }
    OCC_TRY(mark(5));
    // Algorithms 6-7: SFD -> EPD, SwiGLU, weight modulation
    UpArgs up{};
    up.A = x_sfd;
    up.a_rows = bb.epd_src;
    up.Wg = w_gate;
    up.Wu = w_up;
    up.seg_off = bb.epd_off;
    up.tile_off = bb.tile_off;
    up.row_w = bb.epd_w;
    up.out = epd;
    up.gu_out = (D.flags & OCC_FLAG_TRAIN) ? at<void>(workspace, L.gu) : nullptr;
    up.M = D.T * D.k;
    up.K = D.d;
    up.N = D.F;
    up.Ne = D.Ne;
    up.tab = tab;
    OCC_HIP(ops.up(up, routed_tiles, s));
    OCC_TRY(mark(6));
    // Algorithm 8: EPD -> SFD, summed inside each group in fp32.  The first
    // contributor to every SFD row stores (so no zero-fill is needed), then
    // the other rows of the group add with atomics.  Small batches are bound
    // by reading the weights, which the two launches would read twice: there
    // the SFD rows were zeroed by the dispatch and one launch adds every row.
    DownArgs dn{};
    dn.A = epd;
    dn.W = w_down;
    dn.seg_off = bb.epd_off;
    dn.rows = bb.down_rows;
    dn.first_cnt = bb.first_cnt;
    dn.dst_rows = bb.epd_src;
    dn.out = sfd_out;
    dn.M = D.T * D.k;
    dn.K = D.F;
    dn.N = D.d;
    dn.Ne = D.Ne;
    dn.k_split = D.F;
    dn.tab = tab;
    if (det) {
        // first contributors store into their SFD rows, the others at their
        // own EPD rows; the merge then adds those to the SFD rows in slot order
        float *y_epd = at<float>(workspace, L.y_epd);
        dn.epd_out = y_epd;
        dn.phase = 3;
        dn.tile_off = bb.tile_off;
        OCC_HIP(ops.down(dn, routed_tiles, s));
        OCC_TRY(mark(7));
        // stage one (SFD rows) and, in the same pass over each token, stage
        // two (Algorithm 9) with the combine's order of additions
        OCC_HIP(launch_merge_slots(y_epd, ids, bb.tok_epd, bb.brim0, tab, D.T, D.k, D.d, sfd_out,
                                   y_sh, y, bf16, s));
    } else if (one_launch) {
        dn.phase = 0;
        dn.tile_off = bb.tile_off;
        OCC_HIP(ops.down(dn, routed_tiles, s));
        OCC_TRY(mark(7));
    } else {
        dn.phase = 1;
        dn.tile_off = bb.tile_off_first;
        OCC_HIP(ops.down(dn, routed_tiles, s));
        OCC_TRY(mark(7));
        dn.phase = 2;
        dn.tile_off = bb.tile_off_rest;
        OCC_HIP(ops.down(dn, routed_tiles, s));
    }
    OCC_TRY(mark(8));
    // Algorithm 9: SFD -> ORI across groups (+ shared experts), cast once
    if (!det) OCC_HIP(launch_combine(sfd_out, bb.brim0, y_sh, D.T, D.Nd, D.d, bf16, y, s));
    OCC_TRY(mark(9));
    return OCC_OK;
}

occ_status occ_moe_forward(const occ_layer_desc *desc, const void *x, const float *logits,
                           const int32_t *placement_host, const void *w_gate, const void *w_up,
                           const void *w_down, const void *ws_gate, const void *ws_up,
                           const void *ws_down, void *y, void *workspace, size_t ws_bytes,
                           void *const *stage_events, void *stream) {
    if (!logits) return OCC_ERR_INVALID_ARG;
    return forward(desc, x, logits, nullptr, nullptr, nullptr, placement_host, w_gate, w_up,
                   w_down, ws_gate, ws_up, ws_down, y, workspace, ws_bytes, stage_events, stream);
}

occ_status occ_moe_forward_noalloc(const occ_layer_desc *desc, const void *x, const float *logits,
                                   const int32_t *placement_host, const void *w_gate,
                                   const void *w_up, const void *w_down, const void *ws_gate,
                                   const void *ws_up, const void *ws_down, void *y,
                                   void *const *stage_events, void *stream) {
    OCC_TRY(check_desc(desc));
    if (!logits) return OCC_ERR_INVALID_ARG;
    // the backward pass reads the training forward's state from a caller
    // workspace, which this variant does not have
    if (desc->flags & OCC_FLAG_TRAIN) return OCC_ERR_UNSUPPORTED;
    if (layout(*desc).total > OCC_NOALLOC_SCRATCH_BYTES) return OCC_ERR_WORKSPACE;
    void *ws = nullptr;
    OCC_TRY(noalloc_scratch(&ws));
    return forward(desc, x, logits, nullptr, nullptr, nullptr, placement_host, w_gate, w_up,
                   w_down, ws_gate, ws_up, ws_down, y, ws, OCC_NOALLOC_SCRATCH_BYTES,
                   stage_events, stream);
}

occ_status occ_moe_forward_gated(const occ_layer_desc *desc, const void *x, const void *w_router,
                                 const int32_t *placement_host, const void *w_gate,
                                 const void *w_up, const void *w_down, const void *ws_gate,
                                 const void *ws_up, const void *ws_down, void *y,
                                 void *workspace, size_t ws_bytes, void *const *stage_events,
                                 void *stream) {
    if (!w_router) return OCC_ERR_INVALID_ARG;
    return forward(desc, x, nullptr, w_router, nullptr, nullptr, placement_host, w_gate, w_up,
                   w_down, ws_gate, ws_up, ws_down, y, workspace, ws_bytes, stage_events, stream);
}

occ_status occ_gate(const occ_layer_desc *desc, const void *x, const void *w_router,
                    float *logits, void *stream) {
    OCC_TRY(check_desc(desc));
    if (!x || !w_router || !logits) return OCC_ERR_INVALID_ARG;
    OCC_HIP(launch_gate(x, w_router, desc->T, desc->d, desc->Ne, desc->dtype == OCC_BF16, logits,
                        static_cast<hipStream_t>(stream)));
    return OCC_OK;
}

occ_status occ_moe_forward_routed(const occ_layer_desc *desc, const void *x, const int32_t *ids,
                                  const float *w, const int32_t *placement_host,
                                  const void *w_gate, const void *w_up, const void *w_down,
                                  const void *ws_gate, const void *ws_up, const void *ws_down,
                                  void *y, void *workspace, size_t ws_bytes,
                                  void *const *stage_events, void *stream) {
    if (!ids || !w) return OCC_ERR_INVALID_ARG;
    return forward(desc, x, nullptr, nullptr, ids, w, placement_host, w_gate, w_up, w_down, ws_gate,
                   ws_up, ws_down, y, workspace, ws_bytes, stage_events, stream);
}

occ_status occ_moe_backward(const occ_layer_desc *desc, const void *dy, const void *x,
                            const float *logits, const int32_t *placement_host,
                            const void *w_gate, const void *w_up, const void *w_down,
                            const void *ws_gate, const void *ws_up, const void *ws_down,
                            void *dx, float *dw_gate, float *dw_up, float *dw_down,
                            float *dws_gate, float *dws_up, float *dws_down, float *dw,
                            float *dlogits, void *workspace, size_t ws_bytes,
                            void *const *stage_events, void *stream) {
    OCC_TRY(check_desc(desc));
    const occ_layer_desc &D = *desc;
    if (!(D.flags & OCC_FLAG_TRAIN)) return OCC_ERR_INVALID_ARG;
    if (!dy || !x || !w_gate || !w_up || !w_down || !dx || !dw_gate || !dw_up || !dw_down)
        return OCC_ERR_INVALID_ARG;
    if (D.n_shared > 0 && (!ws_gate || !ws_up || !ws_down || !dws_gate || !dws_up || !dws_down))
        return OCC_ERR_INVALID_ARG;
    if (dlogits && !logits) return OCC_ERR_INVALID_ARG;
    if (stage_events)
        for (int i = 0; i <= OCC_BSTAGE_COUNT; i++)
            if (!stage_events[i]) return OCC_ERR_INVALID_ARG;
    PlaceTab tab;
    OCC_TRY(make_tab(D, placement_host, &tab));
    const Layout L = layout(D);
    OCC_TRY(check_ws(D, workspace, ws_bytes, L.total));

    hipStream_t s = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) -> occ_status {
        if (!stage_events) return OCC_OK;
        return hip_status(hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), s));
    };
    const size_t es = elem_bytes(D), T = D.T, d = D.d, F = D.F;
    const size_t Nsh = static_cast<size_t>(D.n_shared) * D.F_shared;
    const BrimBufs bb = brim_bufs(workspace, L);
    const void *x_sfd = at<void>(workspace, L.x_sfd);
    const void *h = at<void>(workspace, L.epd);
    void *dy_sfd = at<void>(workspace, L.dy_sfd);
    void *dgu = at<void>(workspace, L.dgu);
    float *dx_sfd = at<float>(workspace, L.dx_sfd);
    float *dw_part = at<float>(workspace, L.dw_part);
    void *zero_row = at<void>(workspace, L.zero_row);
    int32_t *bt_all = at<int32_t>(workspace, L.bt_all);
    int32_t *bt_first = at<int32_t>(workspace, L.bt_first);
    int32_t *bt_rest = at<int32_t>(workspace, L.bt_rest);
    float *dx_sh = D.n_shared > 0 ? at<float>(workspace, L.dx_sh) : nullptr;
    const size_t routed_tiles = (T * D.k + kBwdRowTile - 1) / kBwdRowTile + D.Ne + kBrimMaxFill;
    const bool det = D.flags & OCC_FLAG_DETERMINISTIC;
    const bool one_launch = !det && static_cast<int64_t>(D.T) * D.k < 128ll * D.Ne;

    OCC_TRY(mark(0));
    // row schedules of the input-gradient tiles, a zero row for the tails of
    // K-major operands
    const size_t zero_elems = std::max<size_t>({d, 2 * F, 2 * Nsh, kBwdTile});
    OCC_HIP(launch_fill_i32(static_cast<int32_t *>(zero_row), zero_elems * es / 4, 0, s));
    // the all-rows schedule filled for the SwiGLU backward's ceil(F / 256)
    // column tiles (the input gradient's product runs on the same schedule),
    // where the forward's is filled too (not in the decode regime, whose
    // products stream their weights and gain nothing from more tiles)
    const int bwd_fill = fill_cols(D) > 0 ? static_cast<int>(ceil_div(F, kBwdTile)) : 0;
    OCC_HIP(launch_tile_sched(bb.epd_off, bb.first_cnt, D.Ne, kBwdRowTile, bwd_fill, bt_all,
                              bt_first, bt_rest, s));
    // dy ORI -> SFD: the combine's transpose copies dy into each replica (and
    // zeroes the dx accumulator rows when the merge is one launch of adds)
    OCC_HIP(launch_dispatch(dy, D.T, D.Nd, d * es, bb.brim0, dy_sfd, s,
                            one_launch ? dx_sfd : nullptr, D.d));
    OCC_TRY(mark(1));
    // dh = dy W_d for every EPD row (its SFD row's gradient, BRIM_1), then
    // the SwiGLU and modulation backward
    BwdDgradArgs g1{};
    g1.A = dy_sfd;
    g1.a_rows = bb.epd_src;
    g1.lda = D.d;
    g1.B1 = w_down;
    g1.seg_off = bb.epd_off;
    g1.tile_off = bt_all;
    g1.first_cnt = bb.first_cnt;
    g1.gu = at<void>(workspace, L.gu);
    g1.gu_ld = 2 * D.F;
    g1.gu_uoff = D.F;
    g1.row_w = bb.epd_w;
    g1.out = dgu;
    g1.out_ld = 2 * D.F;
    g1.out_uoff = D.F;
    g1.dw_part = dw_part;
    g1.dw_stride = L.dw_stride;
    g1.N = D.F;
    g1.K = D.d;
    g1.ksplit = D.d;
    g1.Ne = D.Ne;
    g1.epilogue = BWD_EPI_SWIGLU;
    g1.tab = tab;
    OCC_HIP(launch_bwd_dgrad(g1, routed_tiles, s));
    OCC_TRY(mark(2));
    // dx_epd = dg W_g + du W_u, merged into SFD rows inside each group (fp32)
    BwdDgradArgs g2{};
    g2.A = dgu;
    g2.a_rows = bb.down_rows;
    g2.lda = 2 * D.F;
    g2.B1 = w_gate;
    g2.B2 = w_up;
    g2.seg_off = bb.epd_off;
    g2.first_cnt = bb.first_cnt;
    g2.dst_rows = bb.epd_src;
    g2.merge_out = dx_sfd;
    g2.N = D.d;
    g2.K = 2 * D.F;
    g2.ksplit = D.F;
    g2.Ne = D.Ne;
    g2.epilogue = BWD_EPI_MERGE;
    g2.tab = tab;
    if (det) {
        // first contributors store into their SFD rows of dx, the others at
        // their own EPD rows; summed per SFD row in slot order after the
        // shared experts, with the combine
        g2.epd_out = at<float>(workspace, L.y_epd);
        g2.split = 1;
        g2.phase = 0;
        g2.tile_off = bt_all;
        g2.merge_store = 1;
        OCC_HIP(launch_bwd_dgrad(g2, routed_tiles, s));
    } else if (one_launch) {
        g2.phase = 0;
        g2.tile_off = bt_all;
        g2.merge_store = 0;
        OCC_HIP(launch_bwd_dgrad(g2, routed_tiles, s));
    } else {
        g2.phase = 1;
        g2.tile_off = bt_first;
        g2.merge_store = 1;
        OCC_HIP(launch_bwd_dgrad(g2, routed_tiles, s));
        g2.phase = 2;
        g2.tile_off = bt_rest;
        g2.merge_store = 0;
        OCC_HIP(launch_bwd_dgrad(g2, routed_tiles, s));
    }
    OCC_TRY(mark(3));
    // shared experts: dense over the T tokens, one expert at a time for the
    // input gradients, all at once for the weight gradients
    if (D.n_shared > 0) {
        int32_t *dseg = at<int32_t>(workspace, L.dense_seg);
        int32_t *dtile = at<int32_t>(workspace, L.dense_tile);
        // the row-tile schedule of dh -> dg, du against F_shared columns,
        // balanced over the CUs' rounds (dx_sh below schedules its own)
        const int m_gu = dense_row_tiles_bwd(D.T, ceil_div(D.F_shared, kBwdTile));
        OCC_HIP(launch_dense_sched(D.T, m_gu, dseg, dtile, s));
        PlaceTab one{};
        one.Ne = 1;
        one.Nd = 1;
        one.n = 1;
        void *dgu_sh = at<void>(workspace, L.dgu_sh);
        // the shared W_d transposed (F_shared x d per expert), so that
        // dh_sh = dy W_d reads both operands K-contiguous.  (The routed
        // experts keep transpose reads: there the copy of all their W_d
        // costs what the faster product saves.)
        void *wt_down = at<void>(workspace, L.wt_down);
        OCC_HIP(launch_transpose_bf16(ws_down, D.d, D.F_shared, d * D.F_shared, wt_down, D.d,
                                      static_cast<size_t>(D.F_shared) * d, D.n_shared, s));
        for (int sx = 0; sx < D.n_shared; sx++) {
            const size_t Fs = D.F_shared;
            BwdDgradArgs s1{};
            s1.A = dy;
            s1.lda = D.d;
            s1.B1 = static_cast<const char *>(wt_down) + sx * Fs * d * es;
            s1.b_kcontig = 1;
            s1.seg_off = dseg;
            s1.tile_off = dtile;
            s1.gu = at<void>(workspace, L.gu_sh);
            s1.gu_ld = static_cast<int>(2 * Nsh);
            s1.gu_col = static_cast<int>(sx * Fs);
            s1.gu_uoff = static_cast<int>(Nsh);
            s1.out = dgu_sh;
            s1.out_ld = static_cast<int>(2 * Nsh);
            s1.out_col = static_cast<int>(sx * 2 * Fs);
            s1.out_uoff = static_cast<int>(Fs);
            s1.N = D.F_shared;
            s1.K = D.d;
            s1.ksplit = D.d;
            s1.Ne = 1;
            s1.epilogue = BWD_EPI_SWIGLU;
            s1.tab = one;
            OCC_HIP(launch_bwd_dgrad(s1, m_gu, s));
        }
        // dx_sh = sum over the shared experts of dg W_g + du W_u: one dense
        // product with K = 2 n_shared F_shared against the weights
        // transposed (expert sx's block holds W_g^T then W_u^T), on the
        // forward's down-projection build, whose operands both have the
        // contraction index contiguous (no LDS transpose reads)
        void *wt_sh = at<void>(workspace, L.wt_sh);
        const size_t Fs = D.F_shared, blk = d * 2 * Fs;
        OCC_HIP(launch_transpose_bf16(ws_gate, D.F_shared, D.d, Fs * d, wt_sh,
                                      static_cast<int>(2 * Fs), blk, D.n_shared, s));
        OCC_HIP(launch_transpose_bf16(ws_up, D.F_shared, D.d, Fs * d,
                                      static_cast<char *>(wt_sh) + Fs * es,
                                      static_cast<int>(2 * Fs), blk, D.n_shared, s));
        DownArgs s2{};
        s2.A = dgu_sh;
        s2.W = wt_sh;
        s2.out = dx_sh;
        s2.M = D.T;
        s2.K = static_cast<int>(2 * Nsh);
        s2.N = D.d;
        s2.Ne = 1;
        s2.k_split = static_cast<int>(2 * Fs);
        s2.tab = one;
        const GemmOps ops = gemm_ops(D);
        if (dense_pipelined(ops, D.T, D.d))
            OCC_HIP(launch_gemm_down_bf16_dense(s2, 0, s));
        else
            OCC_HIP(ops.down(s2, 0, s));
        BwdWgradArgs w3{};
        w3.A = dy;
        w3.lda = D.d;
        w3.B = at<void>(workspace, L.h_sh);
        w3.ldb = static_cast<int>(Nsh);
        w3.b_col_grp = D.F_shared;
        w3.zero_row = zero_row;
        w3.C1 = dws_down;
        w3.M = D.d;
        w3.N = D.F_shared;
        w3.msplit = D.d;
        w3.n_groups = D.n_shared;
        w3.rows = D.T;
        w3.tab = one;
        // K = all T tokens against a small output: split into chunks summed
        // in order (enough tiles for the CUs, still deterministic)
        w3.k_parts = wgrad_k_parts(D.n_shared, D.d, D.F_shared, D.T);
        w3.k_chunk = wgrad_k_chunk(D.T, w3.k_parts);
        w3.part = w3.k_parts > 1 ? at<float>(workspace, L.wg_part) : nullptr;
        OCC_HIP(launch_bwd_wgrad(w3, s));
        BwdWgradArgs w4{};
        w4.A = dgu_sh;
        w4.lda = static_cast<int>(2 * Nsh);
        w4.a_col_grp = 2 * D.F_shared;
        w4.B = x;
        w4.ldb = D.d;
        w4.zero_row = zero_row;
        w4.C1 = dws_gate;
        w4.C2 = dws_up;
        w4.M = 2 * D.F_shared;
        w4.N = D.d;
        w4.msplit = D.F_shared;
        w4.n_groups = D.n_shared;
        w4.rows = D.T;
        w4.tab = one;
        w4.k_parts = wgrad_k_parts(D.n_shared, 2 * D.F_shared, D.d, D.T);
        w4.k_chunk = wgrad_k_chunk(D.T, w4.k_parts);
        w4.part = w4.k_parts > 1 ? at<float>(workspace, L.wg_part) : nullptr;
        OCC_HIP(launch_bwd_wgrad(w4, s));
    }
    OCC_TRY(mark(4));
    // dx: SFD -> ORI, summed across groups (the dispatch's transpose), plus
    // the shared experts' part, cast once
    if (det)
        OCC_HIP(launch_merge_slots(at<float>(workspace, L.y_epd), at<int32_t>(workspace, L.ids),
                                   bb.tok_epd, bb.brim0, tab, D.T, D.k, D.d, dx_sfd, dx_sh, dx,
                                   D.dtype == OCC_BF16, s));
    else
        OCC_HIP(launch_combine(dx_sfd, bb.brim0, dx_sh, D.T, D.Nd, D.d, D.dtype == OCC_BF16, dx,
                               s));
    OCC_TRY(mark(5));
    // dW_d[e] = sum over e's rows of dy_sfd[row's SFD row] (x) h[row]
    BwdWgradArgs w1{};
    w1.A = dy_sfd;
    w1.a_rows = bb.epd_src;
    w1.lda = D.d;
    w1.B = h;
    w1.ldb = D.F;
    w1.seg_off = bb.epd_off;
    w1.zero_row = zero_row;
    w1.C1 = dw_down;
    w1.M = D.d;
    w1.N = D.F;
    w1.msplit = D.d;
    w1.n_groups = D.Ne;
    w1.tab = tab;
    OCC_HIP(launch_bwd_wgrad(w1, s));
    OCC_TRY(mark(6));
    // [dW_g; dW_u][e] = sum over e's rows of [dg; du] (x) x_sfd[row's SFD row]
    BwdWgradArgs w2{};
    w2.A = dgu;
    w2.lda = 2 * D.F;
    w2.B = x_sfd;
    w2.b_rows = bb.epd_src;
    w2.ldb = D.d;
    w2.seg_off = bb.epd_off;
    w2.zero_row = zero_row;
    w2.C1 = dw_gate;
    w2.C2 = dw_up;
    w2.M = 2 * D.F;
    w2.N = D.d;
    w2.msplit = D.F;
    w2.n_groups = D.Ne;
    w2.tab = tab;
    OCC_HIP(launch_bwd_wgrad(w2, s));
    OCC_TRY(mark(7));
    // routing-weight and logit gradients
    if (dw || dlogits)
        OCC_HIP(launch_route_backward(logits, at<int32_t>(workspace, L.ids), bb.tok_epd, dw_part,
                                      L.dw_stride, L.dw_stride, D.T, D.Ne, D.k, dw, dlogits, s));
    OCC_TRY(mark(8));
    return OCC_OK;
}

occ_status occ_coactivation_stats(const occ_layer_desc *desc, const int32_t *ids,
                                  const int32_t *placement_host, int32_t *C, float *P,
                                  int64_t *n_sfd, double *ct, double *intra, void *stream) {
    OCC_TRY(check_desc(desc));
    if (!ids || !C || !P || !n_sfd || !ct || !intra) return OCC_ERR_INVALID_ARG;
    PlaceTab tab;
    OCC_TRY(make_tab(*desc, placement_host, &tab));
    OCC_HIP(launch_coact(ids, desc->T, desc->k, tab, C, P, n_sfd, ct, intra,
                         static_cast<hipStream_t>(stream)));
    return OCC_OK;
}

// Algorithm 1 (paper section 3.2).  The 1/|L| and 1/max C scalings of the
// paper's scores do not change any argmax / argmin, so the integer counts are
// used directly; each unused expert's summed collaboration with all placed
// experts and with the current group is kept up to date as experts are
// placed.
occ_status occ_place_experts(const int32_t *C_host, int32_t Ne, int32_t Nd,
                             int32_t *placement_host) {
    if (!C_host || !placement_host || Ne < 1 || Nd < 1 || Ne % Nd != 0 || Ne > 65536)
        return OCC_ERR_INVALID_ARG;
    const int n = Ne / Nd;
    std::vector<char> used(Ne, 0);
    std::vector<int64_t> with_placed(Ne, 0), with_group(Ne, 0);
    for (int g = 0; g < Nd; g++) {
        std::fill(with_group.begin(), with_group.end(), 0);
        int32_t *Lg = placement_host + static_cast<size_t>(g) * n;
        int len = 0;
        auto push = [&](int e) {
            Lg[len++] = e;
            used[e] = 1;
            const int32_t *row = C_host + static_cast<size_t>(e) * Ne;
            for (int q = 0; q < Ne; q++) {
                with_placed[q] += row[q];
                with_group[q] += row[q];
            }
        };
        if (g == 0 && n >= 2) {
            int bi = 0, bj = 1;
            for (int i = 0; i < Ne; i++)
                for (int j = i + 1; j < Ne; j++)
                    if (C_host[static_cast<size_t>(i) * Ne + j] >
                        C_host[static_cast<size_t>(bi) * Ne + bj]) {
                        bi = i;
                        bj = j;
                    }
            push(bi);
            push(bj);
        } else if (g > 0) {
            int best = -1;
            for (int e = 0; e < Ne; e++)
                if (!used[e] && (best < 0 || with_placed[e] < with_placed[best])) best = e;
            push(best);
        }
        while (len < n) {
            int best = -1;
            for (int e = 0; e < Ne; e++)
                if (!used[e] && (best < 0 || with_group[e] > with_group[best])) best = e;
            push(best);
        }
    }
    return OCC_OK;
}

occ_status occ_events_create(int32_t n, void **events_host) {
    if (n < 0 || (n > 0 && !events_host)) return OCC_ERR_INVALID_ARG;
    for (int i = 0; i < n; i++) {
        hipEvent_t e;
        OCC_HIP(hipEventCreate(&e));
        events_host[i] = e;
    }
    return OCC_OK;
}

occ_status occ_events_destroy(int32_t n, void **events_host) {
    if (n < 0 || (n > 0 && !events_host)) return OCC_ERR_INVALID_ARG;
    for (int i = 0; i < n; i++)
        if (events_host[i]) OCC_HIP(hipEventDestroy(static_cast<hipEvent_t>(events_host[i])));
    return OCC_OK;
}

occ_status occ_event_elapsed_ms(void *start, void *stop, float *ms_host) {
    if (!start || !stop || !ms_host) return OCC_ERR_INVALID_ARG;
    OCC_HIP(hipEventSynchronize(static_cast<hipEvent_t>(stop)));
    OCC_HIP(hipEventElapsedTime(ms_host, static_cast<hipEvent_t>(start),
                                static_cast<hipEvent_t>(stop)));
    return OCC_OK;
}

}  // extern "C"
