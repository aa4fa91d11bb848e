/*
 * occ.h -- C ABI of the Occult MoE-layer library for AMD Instinct MI355X (gfx950).
 *
 * The library runs, on one GPU, the data-parallel hot path of the MoE layer of
 * "Occult: Optimizing Collaborative Communication across Experts for
 * Accelerated Parallel MoE Training and Inference" (Luo et al., ICML 2025,
 * arXiv 2505.13345).  The placement's Nd expert groups stand for the Nd
 * devices of expert parallelism; the two all-to-all exchanges of the paper's
 * pipeline (appendix A.1, Algorithm 2) are identities on one GPU, so group g's
 * segment of every SFD buffer is "device g's receive buffer".
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the name ends in _host.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises; all GPU work is queued on `stream` (a hipStream_t, NULL
 *     meaning the null stream) and the call returns at once.
 *   - Arguments are checked on the host before anything is queued.  On any
 *     error nothing is queued and the output buffers are untouched.
 *   - Row-major layouts.  Weights follow nn.Linear (out, in): the reduction
 *     dimension is contiguous.
 *   - Float tensors x, weights and y are all of the descriptor's dtype; router
 *     logits are always fp32.
 *   - Calls are stateless; distinct calls may run concurrently on distinct
 *     streams with distinct workspaces.
 */
#ifndef OCC_H
#define OCC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum occ_status {
    OCC_OK = 0,
    OCC_ERR_INVALID_ARG = 1, /* a null pointer, an impossible shape, a bad placement */
    OCC_ERR_UNSUPPORTED = 2, /* valid, but outside the kernels' limits (see occ_layer_desc) */
    OCC_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or smaller than occ_workspace_size */
    OCC_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} occ_status;

typedef enum occ_dtype { OCC_F32 = 0, OCC_BF16 = 1 } occ_dtype;

/* Collaboration pruning (paper, section 3.3): each token may use experts on
 * at most prune_groups groups.
 * Routing-score-based: the token takes the top k experts, by routing score,
 * among the chosen groups' experts.  The groups are chosen
 *   TRAVERSE: by walking the token's plain top-k experts in descending score
 *             and collecting their groups until prune_groups are reached
 *             (the paper's rule);
 *   GROUPSUM: by ranking the groups that hold at least one plain top-k expert
 *             by the fp32 sum, taken in top-k order, of those experts' logits
 *             (ties to the lower group) and keeping prune_groups of them.
 * Weights stay the full-softmax probabilities (not renormalised).
 * Expert-similarity-based (SIMILARITY, occ_route_similarity only): the groups
 * are chosen as by TRAVERSE; the plain top-k experts in them stay where they
 * are, and each other one, in descending score, is replaced by the first
 * expert of its row of the ranked similarity table (appendix A.3, see
 * occ_similarity_rank) that lies in a chosen group and is not yet selected;
 * the replacement takes over the replaced expert's weight.
 * A token whose plain top k already spans <= prune_groups groups is unchanged
 * under every rule. */
typedef enum occ_prune_rule {
    OCC_PRUNE_OFF = 0,
    OCC_PRUNE_TRAVERSE = 1,
    OCC_PRUNE_GROUPSUM = 2,
    OCC_PRUNE_SIMILARITY = 3
} occ_prune_rule;

/* Training: the forward also keeps what occ_moe_backward needs in the
 * workspace (the SwiGLU pre-activations), and the workspace grows by the
 * backward pass's buffers.  Needs bf16, d >= 256, F >= 256 (and F_shared >=
 * 256 when there are shared experts): OCC_ERR_UNSUPPORTED otherwise. */
#define OCC_FLAG_TRAIN 1

/* Deterministic merge (paper appendix A.2, Algorithm 8, and its remark that
 * the stage-one results may equally be summed serially over the local
 * experts): the down-projection stores each SFD row's first contributor's
 * fp32 result (the token's lowest-position expert in the group) into that
 * row and the other EPD rows' results at their own rows; a pass over each
 * token then adds those to the SFD rows in ascending placement position
 * (slot order inside the group), with no atomic adds, and adds the SFD rows
 * into y (Algorithm 9, in the combine's order).  Every output (y, and with OCC_FLAG_TRAIN every gradient) is then
 * bitwise identical from run to run.  The workspace grows by T*k*d fp32. */
#define OCC_FLAG_DETERMINISTIC 2

/* Shape of one MoE layer.  Limits of the library:
 *   1 <= T, T*k < 2^31;  1 <= Ne <= 256;  1 <= k <= min(Ne, 32);
 *   1 <= Nd <= 64 and Nd divides Ne (n = Ne/Nd experts per group);
 *   bf16: d, F and F_shared multiples of 64;  fp32: multiples of 16;
 *   d <= 8192 (bf16) or 4096 (fp32).
 *   prune_rule != OFF needs prune_groups >= 1 and prune_groups*n >= k. */
typedef struct occ_layer_desc {
    int32_t T;            /* tokens in the batch (ORI rows) */
    int32_t d;            /* hidden size */
    int32_t Ne;           /* routed experts */
    int32_t k;            /* experts per token (top-k) */
    int32_t Nd;           /* expert groups (devices of expert parallelism) */
    int32_t F;            /* routed expert FFN width */
    int32_t n_shared;     /* shared experts, 0 for none */
    int32_t F_shared;     /* shared expert FFN width */
    int32_t prune_rule;   /* occ_prune_rule */
    int32_t prune_groups; /* groups a token may use when pruning */
    int32_t dtype;        /* occ_dtype of x, weights and y */
    int32_t flags;        /* 0, or OCC_FLAG_TRAIN | OCC_FLAG_DETERMINISTIC */
} occ_layer_desc;

/* Index structures of the paper's appendix A.2, as left in the workspace by
 * occ_build_brim / occ_moe_forward.  All device pointers, int32 unless noted.
 *   brim0    Nd x T.  BRIM_0 (Algorithm 3): entry [g, t] is the SFD row holding
 *            token t's single replica for group g, or -1.  One counter runs
 *            over groups outer and tokens inner.
 *   sfd_off  Nd+1.  Group g's SFD rows are [sfd_off[g], sfd_off[g+1]);
 *            sfd_off[Nd] = N_sfd, the number of replicas (CT = N_sfd / T).
 *   epd_off  Ne+1, indexed by placement position p = g*n + j (expert
 *            placement[g][j]): that expert's EPD rows are
 *            [epd_off[p], epd_off[p+1]).  EPD rows are the token replicas
 *            seen by one expert each; there are exactly T*k of them.
 *   epd_src  T*k.  SFD row of each EPD row (the condensed, CSR form of
 *            BRIM_1: row p of BRIM_1 lists exactly these SFD rows).
 *   epd_w    T*k, fp32.  Routing weight of each EPD row.
 *   tok_epd  T*k.  EPD row of token t's j-th routed expert, at t*k + j.
 *   brim1    BRIM_1 (Algorithm 5) as dense matrices, one per group: group g's
 *            block is n x N_g (N_g = sfd_off[g+1]-sfd_off[g]) at offset
 *            n*sfd_off[g]; entry [j, t'] is the group-local EPD row of SFD
 *            row sfd_off[g]+t' for the group's j-th expert, or -1.  A counter
 *            restarts per group and runs over local experts outer, SFD rows
 *            inner.  Written only when dense BRIM_1 is requested.
 *   down_rows T*k.  Each expert's EPD rows reordered for the merge of
 *            Algorithm 8: first the rows that are the first contributor to
 *            their SFD row (the token's lowest-slot expert in that group),
 *            then the others, each in token order; expert p's rows occupy
 *            [epd_off[p], epd_off[p+1]) and the first first_cnt[p] of them
 *            are first contributors.
 *   first_cnt Ne, indexed by placement position.
 *   tile_off Ne+1.  Row-tile schedule of the grouped GEMMs (internal):
 *            position p's row tiles are [tile_off[p], tile_off[p+1]), at
 *            least ceil(rows / tile capacity) of them, more where that fills
 *            the up-projection's last round of the GPU's compute units. */
typedef struct occ_brim {
    int32_t *brim0;
    int32_t *sfd_off;
    int32_t *epd_off;
    int32_t *epd_src;
    float *epd_w;
    int32_t *tok_epd;
    int32_t *brim1;
    int32_t *down_rows;
    int32_t *first_cnt;
    int32_t *tile_off;
} occ_brim;

/* Where occ_moe_forward leaves its intermediate tensors in the workspace.
 *   logits    T x Ne fp32: the router logits, written only by
 *             occ_moe_forward_gated.
 *   ids, w    T x k routing result (int32 / fp32).
 *   x_sfd     N_sfd x d, dtype: the dispatched replicas (ORI -> SFD).
 *   epd       T*k x F, dtype: modulated SwiGLU hidden states (SFD -> EPD).
 *   sfd_out   N_sfd x d, fp32: stage-one sums inside each group (EPD -> SFD).
 *   h_shared  T x n_shared*F_shared, dtype; y_shared T x d, fp32 (or NULL). */
typedef struct occ_forward_view {
    float *logits;
    int32_t *ids;
    float *w;
    occ_brim brim;
    void *x_sfd;
    void *epd;
    float *sfd_out;
    void *h_shared;
    float *y_shared;
} occ_forward_view;

/* Stages timed by occ_moe_forward when given events (see there). */
enum {
    OCC_STAGE_ROUTE = 0,
    OCC_STAGE_BRIM = 1,
    OCC_STAGE_DISPATCH = 2,
    OCC_STAGE_SHARED_UP = 3,       /* shared experts' SwiGLU up-projection
                                      (empty when n_shared = 0) */
    OCC_STAGE_SHARED_DOWN = 4,     /* shared experts' down-projection */
    OCC_STAGE_GEMM_UP = 5,
    OCC_STAGE_GEMM_DOWN_FIRST = 6, /* first contributors, plain stores (one-launch
                                      merge: every row's atomic add;
                                      OCC_FLAG_DETERMINISTIC: every row's
                                      result stored, first contributors'
                                      into their SFD rows) */
    OCC_STAGE_GEMM_DOWN_REST = 7,  /* the other rows, fp32 atomic adds (one-launch
                                      merge: empty; OCC_FLAG_DETERMINISTIC:
                                      the merge and the combine) */
    OCC_STAGE_COMBINE = 8,         /* OCC_FLAG_DETERMINISTIC: empty */
    OCC_STAGE_COUNT = 9
};

/* A fixed string naming the status.  Never NULL. */
const char *occ_status_string(occ_status status);

/* Bytes of device workspace occ_moe_forward needs for this shape (enough for
 * every other call too).  It is sized for the worst case N_sfd = T*min(k, Nd),
 * so no call ever has to read a data-dependent size back to the host.
 * Errors: INVALID_ARG / UNSUPPORTED as for the other calls. */
occ_status occ_workspace_size(const occ_layer_desc *desc, size_t *bytes_host);

/* Router, paper Eq. 2 (section 2.1): R(x) = Top-K(Softmax(g(x)), k), with the
 * logits g(x) given, plus optional collaboration pruning (section 3.3; see
 * occ_prune_rule).
 *   logits           T x Ne fp32.
 *   placement_host   Nd x n int32 in host memory: group g holds experts
 *                    placement_host[g*n + 0 .. g*n + n-1]; must be a
 *                    permutation of 0..Ne-1 (used only when pruning).
 *   ids  (out)       T x k int32: the token's experts, in descending logit
 *                    order, ties to the lower expert index.
 *   w    (out)       T x k fp32: their softmax probabilities over all Ne
 *                    logits, not renormalised.
 * A NaN logit ranks as -inf (the ids stay distinct and in range; the weights
 * are then unspecified).  prune_rule SIMILARITY needs the table: use
 * occ_route_similarity (INVALID_ARG here). */
occ_status occ_route(const occ_layer_desc *desc, const float *logits,
                     const int32_t *placement_host, int32_t *ids, float *w, void *stream);

/* Expert similarity table, paper appendix A.3, Eq. 6-8, built from profiled
 * router logits H (tokens x Ne) in batches.
 * occ_similarity_accumulate adds one batch to the Gram matrix of H's columns:
 *   gram[i][j] += sum over the batch's tokens t of H[t][i] * H[t][j],
 * in fp64, each entry summed in ascending token order (the fp32 products are
 * exact in fp64, so the result does not depend on the launch shape).
 *   T            tokens in this batch (0 is a no-op);  1 <= Ne <= 256.
 *   logits       T x Ne fp32 (device).
 *   gram         Ne x Ne fp64 (device, in/out); zero it before the first batch.
 * Errors: INVALID_ARG for a NULL pointer or a bad size. */
occ_status occ_similarity_accumulate(int32_t T, int32_t Ne, const float *logits, double *gram,
                                     void *stream);

/* The table from an accumulated Gram matrix.  Eq. 7 (Eq. 8 equals it: its
 * 1/N factors cancel): t2[i][j] = gram[i][j]^2 / (gram[i][i] * gram[j][j]),
 * 0 when either column was all zero.  The paper declares the table integer;
 * it is read as each row's ranking: rank[i][q] is the q-th most similar
 * expert to i by t2 descending, ties to the lower index, so every row is a
 * permutation of 0..Ne-1 (and starts with i unless i's column was zero).
 *   gram   Ne x Ne fp64 (device);  t2 (out) Ne x Ne fp64 or NULL;
 *   rank (out) Ne x Ne int32 (device). */
occ_status occ_similarity_rank(int32_t Ne, const double *gram, double *t2, int32_t *rank,
                               void *stream);

/* Router with expert-similarity-based collaboration pruning (section 3.3,
 * see occ_prune_rule).  desc->prune_rule must be OCC_PRUNE_SIMILARITY.
 * Arguments as occ_route, plus
 *   sim_rank   Ne x Ne int32 (device), as written by occ_similarity_rank;
 *              each row must be a permutation of 0..Ne-1 (otherwise the ids
 *              are unspecified but in range).
 * ids keep the plain top-k order (a replacement sits at the replaced
 * expert's place) and w the plain top-k weights. */
occ_status occ_route_similarity(const occ_layer_desc *desc, const float *logits,
                                const int32_t *placement_host, const int32_t *sim_rank,
                                int32_t *ids, float *w, void *stream);

/* BRIM_0 and BRIM_1, paper appendix A.2 (Algorithms 3 and 5), from routing
 * ids/w (T x k, as written by occ_route) and the placement (host, as above).
 * Writes the structures of occ_brim into `workspace` (ws_bytes >=
 * occ_workspace_size) and returns their device addresses in *out_host.
 * dense_brim1 != 0 also writes the dense BRIM_1 matrices.  The routing is
 * first copied into the workspace (occ_forward_views: ids, w), where a
 * token's id outside 0..Ne-1 or repeating an earlier one is replaced by the
 * lowest expert not in its list, with weight 0; valid routing is copied
 * unchanged. */
occ_status occ_build_brim(const occ_layer_desc *desc, const int32_t *ids, const float *w,
                          const int32_t *placement_host, int dense_brim1, void *workspace,
                          size_t ws_bytes, occ_brim *out_host, void *stream);

/* The whole layer, paper Eq. 1 through the pipeline of Algorithm 2:
 *   route (Eq. 2) -> BRIM_0/BRIM_1 -> dispatch ORI->SFD (Alg. 4) ->
 *   SwiGLU up-projection SFD->EPD with the routing weight applied to the
 *   hidden state (Alg. 6-7) -> down-projection EPD->SFD summed inside each
 *   group in fp32 (Alg. 8: the first contributor to each SFD row stores, the
 *   others add; when T*k < 128*Ne the SFD rows are zeroed and every row
 *   adds, in one launch) -> combine SFD->ORI summed across groups (Alg. 9).
 * Without pruning the result equals the plain top-k MoE output (section 3.2).
 *   x          T x d (dtype);  logits T x Ne fp32;  placement_host as above.
 *   w_gate     Ne x F x d;  w_up Ne x F x d;  w_down Ne x d x F (dtype).
 *   ws_gate    n_shared x F_shared x d, ws_up likewise, ws_down
 *              n_shared x d x F_shared: shared experts, dense and ungated,
 *              added with weight 1; NULL when n_shared = 0.
 *   y (out)    T x d (dtype).
 *   workspace  device, 256-byte aligned, ws_bytes >= occ_workspace_size;
 *              holds the intermediates afterwards (occ_forward_views).
 *   stage_events  NULL, or OCC_STAGE_COUNT+1 hipEvent_t handles: event 0 is
 *              recorded on `stream` before the first stage and event s+1
 *              right after stage s, so the pair (s, s+1) times stage s. */
occ_status occ_moe_forward(const occ_layer_desc *desc, const void *x, const float *logits,
                           const int32_t *placement_host, const void *w_gate, const void *w_up,
                           const void *w_down, const void *ws_gate, const void *ws_up,
                           const void *ws_down, void *y, void *workspace, size_t ws_bytes,
                           void *const *stage_events, void *stream);

/* Gate projection g(x) of the router (section 2.1: a single linear layer):
 *   logits[t][e] = sum_i x[t][i] * w_router[e][i], accumulated in fp32
 * (bf16: matrix-core products of the exact bf16 inputs, one accumulation
 * chain per logit in fixed order).
 *   x          T x d (dtype, device);  w_router Ne x d (dtype, device).
 *   logits     (out) T x Ne fp32 (device). */
occ_status occ_gate(const occ_layer_desc *desc, const void *x, const void *w_router,
                    float *logits, void *stream);

/* The layer with the gate projection in front of the router (the decode
 * path: logits are not an input): occ_gate into the workspace (view
 * `logits`), then occ_moe_forward on those logits.  The route stage's events
 * time both.  Arguments as occ_moe_forward, with w_router (Ne x d, dtype)
 * in place of logits; the SIMILARITY rule is not available here. */
occ_status occ_moe_forward_gated(const occ_layer_desc *desc, const void *x, const void *w_router,
                                 const int32_t *placement_host, const void *w_gate,
                                 const void *w_up, const void *w_down, const void *ws_gate,
                                 const void *ws_up, const void *ws_down, void *y,
                                 void *workspace, size_t ws_bytes, void *const *stage_events,
                                 void *stream);

/* The layer from a routing computed elsewhere (for instance by
 * occ_route_similarity): occ_moe_forward without its router stage.
 *   ids, w   T x k int32 / fp32 (device): each token's experts and weights;
 *            sanitised into the workspace as for occ_build_brim.
 * Other arguments as occ_moe_forward; desc->prune_rule is not used.  The
 * route stage's events time that copy. */
occ_status occ_moe_forward_routed(const occ_layer_desc *desc, const void *x, const int32_t *ids,
                                  const float *w, const int32_t *placement_host,
                                  const void *w_gate, const void *w_up, const void *w_down,
                                  const void *ws_gate, const void *ws_up, const void *ws_down,
                                  void *y, void *workspace, size_t ws_bytes,
                                  void *const *stage_events, void *stream);

/* Bytes of the device array that occ_moe_forward_noalloc uses as its
 * workspace (128 MiB, held on every GPU the library runs on until the
 * process ends). */
#define OCC_NOALLOC_SCRATCH_BYTES (128u << 20)

/* occ_moe_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the intermediates live in a static
 * device array of OCC_NOALLOC_SCRATCH_BYTES, one per GPU.  Nothing is
 * allocated or freed; the caller still passes inputs and outputs, with the
 * meaning, layouts and stream semantics of occ_moe_forward.  Shapes whose
 * occ_workspace_size exceeds OCC_NOALLOC_SCRATCH_BYTES return
 * OCC_ERR_WORKSPACE (e.g. the OLMoE shape, d = 2048, 64 experts of F = 1024,
 * top-8, fits up to about 1,100 tokens, or 700 with
 * OCC_FLAG_DETERMINISTIC); OCC_FLAG_TRAIN returns OCC_ERR_UNSUPPORTED (the
 * backward pass reads its state from a caller workspace).  The first call on
 * a GPU looks up the array's device address there; later calls reuse it.
 * All calls on one GPU share that GPU's array and it keeps the last call's
 * contents: calls that may overlap on one GPU (several streams or host
 * threads) race and must be ordered by the caller.  The intermediates are
 * not exposed (occ_forward_views needs a caller workspace). */
occ_status occ_moe_forward_noalloc(const occ_layer_desc *desc, const void *x, const float *logits,
                                   const int32_t *placement_host, const void *w_gate,
                                   const void *w_up, const void *w_down, const void *ws_gate,
                                   const void *ws_up, const void *ws_down, void *y,
                                   void *const *stage_events, void *stream);

/* Stages timed by occ_moe_backward when given events. */
enum {
    OCC_BSTAGE_DISPATCH = 0,    /* dy ORI -> SFD (BRIM_0) */
    OCC_BSTAGE_DGRAD_DOWN = 1,  /* dh = dy W_d per EPD row, SwiGLU backward */
    OCC_BSTAGE_DGRAD_UP = 2,    /* dg W_g + du W_u, merged EPD -> SFD in fp32
                                   (OCC_FLAG_DETERMINISTIC: stored per EPD
                                   row, merged in the combine stage) */
    OCC_BSTAGE_SHARED = 3,      /* the shared experts' four products */
    OCC_BSTAGE_COMBINE = 4,     /* dx SFD -> ORI across groups (+ shared);
                                   OCC_FLAG_DETERMINISTIC: the slot-order
                                   merge too */
    OCC_BSTAGE_WGRAD_DOWN = 5,  /* dW_d = sum dy h^T per expert */
    OCC_BSTAGE_WGRAD_UP = 6,    /* dW_g, dW_u = sum [dg; du] x^T per expert */
    OCC_BSTAGE_ROUTE = 7,       /* routing-weight and logit gradients */
    OCC_BSTAGE_COUNT = 8
};

/* Backward pass of the layer (the training the paper runs, sections 1 and
 * 4.3; its sparse matrix products serve "both forward and backward passes").
 * The routing ids are held fixed; with dy the gradient of the loss in y:
 *   per EPD row (token t, expert e, weight w, a = silu(g) u):
 *     dh = W_d[e]^T dy_t,  dw = <dh, a>,  dg = w dh u silu'(g),
 *     du = w dh silu(g),   dx_t += W_g[e]^T dg + W_u[e]^T du,
 *     dW_d[e] += dy_t (w a)^T,  dW_g[e] += dg x_t^T,  dW_u[e] += du x_t^T;
 *   shared experts likewise with w = 1;
 *   dlogits[t][i] = p_i ([i chosen] dw_i - sum_j dw_j p_(e_j)), p the full
 *   softmax of Eq. 2 (the weights are not renormalised).
 * The Occult structure runs in reverse: dy is dispatched to the SFD rows
 * (BRIM_0), each EPD row gathers its SFD row's gradient (BRIM_1), the input
 * gradients of a group's experts are merged into SFD rows in fp32 (first
 * contributor stores, the rest add) and summed across groups into dx.
 *   workspace   must hold the state of an occ_moe_forward / _gated / _routed
 *               call made with desc->flags = OCC_FLAG_TRAIN on the same x,
 *               weights and placement (nothing else may run in between).
 *   dy          T x d (dtype).  x, weights, placement_host: as the forward.
 *   logits      T x Ne fp32 of that forward (the gated forward's are in its
 *               workspace, see occ_forward_views), or NULL: then dlogits
 *               must be NULL.
 *   dx (out)    T x d (dtype), fp32 sums cast once.
 *   dw_gate, dw_up (out)  Ne x F x d fp32;  dw_down (out) Ne x d x F fp32.
 *   dws_gate, dws_up, dws_down (out)  the shared experts' (n_shared x ...),
 *               fp32; NULL when n_shared = 0.
 *   dw (out)    T x k fp32 routing-weight gradients, or NULL.
 *   dlogits (out)  T x Ne fp32, or NULL.
 *   stage_events  NULL or OCC_BSTAGE_COUNT+1 events, as for the forward.
 * Errors: INVALID_ARG (missing pointers, flags without OCC_FLAG_TRAIN),
 * UNSUPPORTED, WORKSPACE, HIP. */
occ_status occ_moe_backward(const occ_layer_desc *desc, const void *dy, const void *x,
                            const float *logits, const int32_t *placement_host,
                            const void *w_gate, const void *w_up, const void *w_down,
                            const void *ws_gate, const void *ws_up, const void *ws_down,
                            void *dx, float *dw_gate, float *dw_up, float *dw_down,
                            float *dws_gate, float *dws_up, float *dws_down, float *dw,
                            float *dlogits, void *workspace, size_t ws_bytes,
                            void *const *stage_events, void *stream);

/* Device addresses of the intermediates occ_moe_forward leaves in a
 * workspace (pure host arithmetic, nothing queued). */
occ_status occ_forward_views(const occ_layer_desc *desc, void *workspace,
                             occ_forward_view *out_host);

/* Co-activation statistics of a routed batch (ids T x k, placement host).
 *   C (out)      Ne x Ne int32, paper Eq. 3: tokens activating both i and j,
 *                over ordered pairs of a token's experts (C[i][i] = load of i).
 *   P (out)      Ne x Ne fp32, Eq. 4: C / max C with the max over i != j,
 *                one correctly rounded fp32 division per entry, P[i][i] = 0
 *                (all zero when no pair exists).
 *   n_sfd (out)  1 int64: replicas, i.e. distinct groups summed over tokens.
 *   ct (out)     1 fp64: CT = n_sfd / T, the mean replicas per token (section
 *                2.2), bounded by Eq. 5: ceil(k*Nd/Ne) <= CT <= min(k, Nd).
 *   intra (out)  1 fp64: share of the off-diagonal co-activations whose two
 *                experts share a group (the Intra / Inter split of Table 1).
 * ids are expected distinct within a token and in 0..Ne-1; an id out of
 * range is counted as expert 0 (unspecified statistics, in-bounds writes). */
occ_status occ_coactivation_stats(const occ_layer_desc *desc, const int32_t *ids,
                                  const int32_t *placement_host, int32_t *C, float *P,
                                  int64_t *n_sfd, double *ct, double *intra, void *stream);

/* Expert placement rescheduling, paper section 3.2, Algorithm 1, on the host
 * (an offline step run once per layer on profiled counts).  C_host: Ne x Ne
 * co-activation counts (as from occ_coactivation_stats, copied to the host).
 * Group 0 is seeded with the most collaborative pair, each later group with
 * the unused expert least collaborative with all placed experts, and each
 * group grows to n = Ne/Nd experts by the unused expert most collaborative
 * with its members; ties go to the lowest index.  Writes Nd x n experts to
 * placement_host in push order. */
occ_status occ_place_experts(const int32_t *C_host, int32_t Ne, int32_t Nd,
                             int32_t *placement_host);

/* Small helpers so callers can time stages without linking HIP themselves:
 * create / destroy n hipEvent_t handles, and read the milliseconds between
 * two recorded events (waits for the second one). */
occ_status occ_events_create(int32_t n, void **events_host);
occ_status occ_events_destroy(int32_t n, void **events_host);
occ_status occ_event_elapsed_ms(void *start, void *stop, float *ms_host);

#ifdef __cplusplus
}
#endif

#endif /* OCC_H */
