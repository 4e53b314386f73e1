// Host-side validation and launch planning (no HIP calls).
#include "dab_plan.h"

#include <math.h>

namespace dab {
namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Plan a row-panel GEMV over `batch` input rows: W [N, K], `rpw` rows per
// wave.  Batch rows go four (or two, or one) to a workgroup, as many as the
// LDS budget for their fp32 copies allows.  With several batch groups the
// panels are padded to a multiple of 8 so that the groups sharing one panel
// of W land on one XCD and read it through its L2 (see panel_decode).
bool plan_panel(int K, int N, int batch, int rpw, PanelPlan* g) {
    g->K = K;
    g->N = N;
    g->mfma = false;
    g->rows_per_wave = rpw;
    g->rows = 4 * rpw;
    if (N % g->rows != 0) return false;
    g->panels = N / g->rows;
    int nb = batch <= 1 ? 1 : batch == 2 ? 2 : 4;
    while (nb > 1 && (size_t)nb * K * sizeof(float) > (size_t)kPanelLds) nb >>= 1;
    if ((size_t)nb * K * sizeof(float) > (size_t)kPanelLds) return false;
    g->nb = nb;
    g->nbg = ceil_div(batch, nb);
    g->grid = g->nbg == 1 ? g->panels : (int)align_up((size_t)g->panels, 8) * g->nbg;
    g->lds = (size_t)nb * K * sizeof(float);
    return true;
}

// An MFMA panel (bf16): one or two 16-row tiles x all K for 16 or 32
// sequences, in stages of 512 K values (the last one partial where K is not
// a multiple of 512); for QKV a tile is 8 RoPE pairs of one head.  32
// sequences per workgroup (two groups of 16) above a batch of 16, so that
// every weight byte is read by one workgroup; two tiles share each batch
// operand where that still leaves at least 256 workgroups (one per CU) and
// the groups are one, else one tile (more workgroups, each with less LDS).
bool plan_mfma_panel(int K, int N, int batch, bool qkv, int half, PanelPlan* g) {
    if (K % 8 != 0 || N % 16 != 0 || (qkv && half % 8 != 0)) return false;
    const int ng = batch > 16 ? 2 : 1;
    const int nbg = ceil_div(batch, 16 * ng);
    // two tiles: on the streamed and resident-operand panels (16 sequences, K <= 4096, one workgroup
    // per CU) where that still leaves 192 workgroups, on the staged panels where it leaves 256 (fewer
    // measured slower: 8B layer, batch 16, output projection 13.2 -> 19.8 us with 128 two-tile panels;
    // its QKV projection on the streamed panel 16.2 us with 192 two-tile panels, 23.2 us with 384
    // one-tile panels, a round and a half)
    // (The streamed panel, K of 1024, 2048 or 4096, takes two tiles with 32 sequences as well: the GQA
    // layer's ragged batch of 32, QKV projection 25.5 us with 384 one-tile panels, 16.9 us with 192
    // two-tile panels, on MI355X.)
    const bool streamed = K == 1024 || K == 2048 || K == 4096;
    const bool resident = streamed || (ng == 1 && K <= 4096 && K % 256 == 0);
    const bool two = (ng == 1 || streamed) && N % 32 == 0 && (!qkv || half % 16 == 0) &&
                     (long long)(N / 32) * nbg >= (resident ? 192 : 256);
    // QKV on the streamed panel: 24-row panels (three half tiles of 4 RoPE pairs) where they make at
    // most one per CU and more than the 32-row panels would (8B GQA layer: 256 against 192)
    const int cus = 256;
    const bool rows24 = qkv && streamed && half % 4 == 0 && N % 24 == 0 && (long long)(N / 24) * nbg <= cus &&
                        (N / 24) * nbg > (two ? (N / 32) * nbg : (N / 16) * nbg);
    g->K = K;
    g->N = N;
    g->mfma = true;
    g->rows_per_wave = 0;
    g->rows = rows24 ? 24 : two ? 32 : 16;
    g->panels = N / g->rows;
    g->nb = 16 * ng;
    g->nbg = nbg;
    g->grid = g->nbg == 1 ? g->panels : (int)align_up((size_t)g->panels, 8) * g->nbg;
    g->lds = 0;
    return true;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

dab_status make_plan(const dab_config* cfg, Plan* p, int attn_cus, int attn_per_cu) {
    if (!cfg || !p) return DAB_ERR_INVALID_ARG;
    *p = Plan();
    const dab_config& c = *cfg;
    if (c.batch < 0 || c.hidden <= 0 || c.n_q_heads <= 0 || c.n_kv_heads <= 0 || c.head_dim <= 0 ||
        c.cache_capacity <= 0)
        return DAB_ERR_INVALID_ARG;
    if (c.dtype != DAB_F32 && c.dtype != DAB_BF16) return DAB_ERR_INVALID_ARG;
    if (!(c.rope_theta > 0.f) || !isfinite(c.rope_theta) || !(c.eps >= 0.f) || !isfinite(c.eps))
        return DAB_ERR_INVALID_ARG;
    if (c.n_q_heads % c.n_kv_heads != 0) return DAB_ERR_INVALID_ARG;
    if (c.head_dim != 64 && c.head_dim != 128) return DAB_ERR_UNSUPPORTED;
    if (c.hidden % 64 != 0) return DAB_ERR_UNSUPPORTED;
    // every GEMV workgroup keeps one batch row of its input in LDS as fp32
    if ((size_t)c.hidden * sizeof(float) > (size_t)kPanelLds ||
        (size_t)c.n_q_heads * c.head_dim * sizeof(float) > (size_t)kPanelLds)
        return DAB_ERR_UNSUPPORTED;
    if (c.n_q_heads / c.n_kv_heads > kMaxGroup) return DAB_ERR_UNSUPPORTED;
    if (c.kv_chunk != 0 && (c.kv_chunk < 32 || c.kv_chunk > 4096 || c.kv_chunk % 16 != 0))
        return DAB_ERR_INVALID_ARG;
    if (c.max_position < 0 || c.max_position >= c.cache_capacity) return DAB_ERR_INVALID_ARG;
    // keep every element offset of the caches and weights inside int64 and
    // the per-dimension products inside int32
    const long long n_qkv = (long long)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
    if (n_qkv > (1 << 24) || c.hidden > (1 << 20) || c.cache_capacity > (1 << 24) || c.batch > 4096)
        return DAB_ERR_UNSUPPORTED;

    p->B = c.batch;
    p->H = c.hidden;
    p->nq = c.n_q_heads;
    p->nkv = c.n_kv_heads;
    p->D = c.head_dim;
    p->cap = c.cache_capacity;
    p->pos_end = c.max_position > 0 ? c.max_position + 1 : c.cache_capacity;
    p->dtype = c.dtype;
    p->G = c.n_q_heads / c.n_kv_heads;
    p->n_qkv = (int)n_qkv;
    p->n_q = c.n_q_heads * c.head_dim;
    p->theta = c.rope_theta;
    p->eps = c.eps;
    p->elem = c.dtype == DAB_BF16 ? 2 : 4;

    const int B = p->B > 0 ? p->B : 1;  // plan a batch-0 call as batch 1; nothing is launched

    if (c.schedule < DAB_SCHEDULE_AUTO || c.schedule > DAB_SCHEDULE_FUSED) return DAB_ERR_INVALID_ARG;

    // the one-launch kernels are instantiated for groups 1, 2, 4, 8 and for
    // projections of whole K-blocks (4096 bf16 or 2048 fp32 values): the
    // output projection's K (nq D) for attention + projection, the QKV
    // projection's K (H) for QKV + attention
    const int kblock = 64 * 8 * (16 / p->elem);
    const bool group_ok = p->G == 1 || p->G == 2 || p->G == 4 || p->G == 8;
    p->attn_oproj_ok = group_ok && p->n_q % kblock == 0;
    p->qkv_attn_ok = group_ok && p->H % kblock == 0;
    // the whole step in one launch: the output projection's panels as in the
    // one-launch attention + projection, the QKV panels of any width, batches
    // of up to 4 held by one workgroup in both projections (their fp32 input
    // rows within the LDS budget)
    const int nb_all = B <= 1 ? 1 : B == 2 ? 2 : 4;
    const int kmax = p->H > p->n_q ? p->H : p->n_q;
    p->fused_ok = group_ok && p->n_q % kblock == 0 && B <= 4 &&
                  (size_t)nb_all * kmax * sizeof(float) <= (size_t)kPanelLds;
    if ((c.schedule == DAB_SCHEDULE_ATTN_OPROJ && !p->attn_oproj_ok) ||
        (c.schedule == DAB_SCHEDULE_QKV_ATTN && !p->qkv_attn_ok) ||
        (c.schedule == DAB_SCHEDULE_FUSED && !p->fused_ok))
        return DAB_ERR_UNSUPPORTED;
    // AUTO: the schedule measured fastest on MI355X.  Attention + projection
    // in one launch wins for one query head per kv head at small batch (7B
    // layer, batch 1: 42.7 against 43.7 us at 4K tokens, 38.6 against 39.6
    // at 1K); with grouped heads the attention chunks run two to a CU and
    // the waiting projection workgroups cost them slots (8B GQA layer: 267
    // against 169 us at batch 16, 71.9 against 69.8 at batch 1 and 16K
    // tokens).  QKV + attention in one launch never won: the early K/V loads
    // delay the QKV weight stream that every chunk waits for.  The whole step
    // in one launch measured 43.5 against 42.0 us (7B layer, batch 1, 4K
    // tokens): its attention chunks get slots only as QKV panels finish, so
    // they start over 8 us instead of together, and the last of them ends
    // later; with the chunks placed before the k and v panels (so that they
    // start at once) the 512 chunks waiting for q held half the slots and the
    // step took 76 us.
    const bool auto_attn_oproj = p->attn_oproj_ok && p->G == 1 && B <= 4;
    p->schedule = c.schedule != DAB_SCHEDULE_AUTO ? c.schedule
                : auto_attn_oproj ? DAB_SCHEDULE_ATTN_OPROJ : DAB_SCHEDULE_PHASED;

    // projections.  VALU panels: QKV with one RoPE pair (rows e and e + D/2
    // of a head) per wave, the output projection with one row per wave
    // (twice the workgroups for a quarter of the stream).  In the phased
    // schedule, bf16 batches of 8 or more take MFMA panels instead (16
    // sequences per workgroup: the VALU panel holds 4 and would read each
    // panel of weights once per group of 4).
    const bool mfma = p->schedule == DAB_SCHEDULE_PHASED && p->dtype == DAB_BF16 && B >= 8;
    const int half = p->D / 2;
    if (!(mfma && plan_mfma_panel(p->H, p->n_qkv, B, true, half, &p->qkv)) && !plan_panel(p->H, p->n_qkv, B, 2, &p->qkv))
        return DAB_ERR_UNSUPPORTED;
    // In the one-launch attention + projection, two rows per wave: half the
    // projection workgroups, so that with ~512 attention chunks all of them
    // hold a slot from the start and their weights stream with the cache
    // (with 1024, the last ones got slots only as chunks finished and their
    // weight loads ended the step).
    const int rpw_o = p->schedule == DAB_SCHEDULE_ATTN_OPROJ || p->schedule == DAB_SCHEDULE_FUSED ? 2 : 1;
    if (!(mfma && plan_mfma_panel(p->n_q, p->H, B, false, half, &p->oproj)) &&
        !plan_panel(p->n_q, p->H, B, rpw_o, &p->oproj))
        return DAB_ERR_UNSUPPORTED;

    // split-KV chunk over the cached tokens (at most cap - 1; the new token
    // rides with the last chunk): about 512 chunks per pass over the batch
    // and kv heads (two per CU: measured faster than 1024 at 1K and 4K
    // tokens on the 7B layer, and it leaves slots for the projection in the
    // one-launch schedule), at most 64 per (sequence, kv head) so that the
    // merge stays short, in steps of 16 tokens, at least one buffer of loads
    // (256 / (D/8) row slots x 4 tokens) and at most 448 tokens, which keeps
    // ragged batches balanced (GQA layer, batch 32, lengths U[256, 8192]:
    // chunks of 448 tokens 169.9 us per step, 512 tokens 176.7 us with the
    // same merge kernel, on MI355X); longer only where the context would need
    // more than kMaxChunks chunks.  The history is what the positions in use
    // can hold: below the max_position hint where one is given, so that a
    // cache much larger than its sequences provisions no empty workgroups
    // (8B GQA layer, batch 16, 4K tokens in a cache of 16384: 99.2 against
    // 74.6 us per step at capacity 4097, on MI355X).
    const int hist = p->pos_end - 1 > 0 ? p->pos_end - 1 : 1;
    ChunkRule& r = p->chunk;
    r.fixed = c.kv_chunk;
    if (r.fixed == 0) {
        const int half_batch = 256 / (p->D / 8) * 4;
        int want = ceil_div(512, (long long)B * p->nkv);              // chunks per sequence and kv head
        if (want > 64) want = 64;
        r.want = want;
        r.lo = half_batch;
        r.hi = 448;
        // With a (sequence, kv head) pair for every CU already, a short
        // sequence is not split (its chunks would only add merge work), long
        // ones take chunks of at most 384 tokens, and the two-per-CU rule
        // below stays off (it would give the ragged batch's sequences of
        // 1-2K tokens chunks of up to 1024, which finish last).  GQA layer,
        // batch 32, lengths U[256, 8192], on MI355X: at least two chunks of
        // at most 448 tokens (two-per-CU rule on) 147.8 us per step; every
        // sequence in chunks of 448, 384, 352 or 320 tokens 146.2, 144.6,
        // 145.2, 145.4 us; 384 with the two-per-CU rule on 157.2 us.
        const bool pair_per_cu = (long long)B * p->nkv >= 256;
        if (pair_per_cu) {
            r.want = 1;
            r.hi = 384;
        }
        // One query head per kv head: an attention workgroup loads one whole
        // buffer of 256 / (D/8) x 8 tokens per round trip, so a chunk is a
        // whole number of buffers (7B layer, batch 1, 1K tokens: 64-token
        // chunks 34.9 us, 128-token chunks 33.7 us per step on MI355X; at 4K
        // the 256 tokens of the rule above are two buffers already).
        r.whole = p->G == 1 ? 2 * half_batch : 16;
        r.maxc = kMaxChunks;
        int T = chunk_len(r, hist);
        // Phased schedule: where those chunks need more than one round of the
        // attention kernel's resident workgroups, take two chunks per CU (all
        // resident at once) if that still gives every (sequence, kv head) a
        // chunk, up to 1024 tokens a chunk; longer chunks would unbalance
        // ragged batches.  (8B GQA layer, batch 16, 4K tokens, four attention
        // workgroups resident per CU, on MI355X: 512 chunks of 1024 tokens
        // 86.4 us per step, 768 of 688 86.9, 1024 of 512 89.0, partial rounds
        // of 640 or 896 chunks 91-94.)
        // (The rule is evaluated again at every sequence's position, so the
        // round count is judged for the tokens the sequences hold.)
        const long long pairs = (long long)B * p->nkv;
        const long long two_per_cu = 2LL * attn_cus;
        if (p->schedule == DAB_SCHEDULE_PHASED && attn_cus > 0 && attn_per_cu >= 2 && pairs <= two_per_cu &&
            !pair_per_cu) {
            r.want2 = (int)(two_per_cu / pairs);
            r.hi2 = 1024;
            r.pairs = (int)pairs;
            r.resident = attn_cus * attn_per_cu;
            T = chunk_len(r, hist);
        }
        while (ceil_div(hist, T) > kMaxChunks) T += 512;
        r.maxc = ceil_div(hist, T);
    } else {
        r.maxc = ceil_div(hist, r.fixed);
    }
    const int T = chunk_len(r, hist);
    p->kv_chunk = T;
    p->max_chunks = r.maxc;
    if (p->max_chunks > kMaxChunks) return DAB_ERR_UNSUPPORTED;
    const long long attn_grid = (long long)B * p->nkv * p->max_chunks;
    if (attn_grid + p->qkv.grid + p->oproj.grid > (1LL << 30)) return DAB_ERR_UNSUPPORTED;
    p->attn_grid = (int)attn_grid;
    // The last chunk of a (sequence, kv group) merges G heads x chunks
    // partials with device-coherent loads, merge_round(G) chunks per thread
    // and head at a time; each round costs ~2-3 us on MI355X with the
    // launch otherwise idle (a GQA layer at 16K tokens, 64 chunks of 4
    // heads: four rounds, a 10 us tail behind 8 workgroups).  Where one
    // round does not cover the chunks, the phased schedule merges in a
    // kernel of its own instead: plain loads after the kernel boundary, one
    // workgroup per (sequence, q head), every load of a round in flight.
    p->split_merge = p->schedule == DAB_SCHEDULE_PHASED &&
                     ceil_div(p->max_chunks, 256 / p->D) > merge_round(p->G);

    // workspace layout
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    p->off_flags = take(256);
    p->off_attn_cnt = take(sizeof(int32_t) * B * p->nkv);
    p->off_seq_ready = take(sizeof(int32_t) * B * kReadyCopies * kReadyStride);
    p->off_ready_done = take(sizeof(int32_t) * B * kReadyCopies * kReadyStride);
    // panel counts per (batch group, head) (QKV + attention) or per (sequence, head) (whole step)
    p->off_head_cnt = take(sizeof(int32_t) * B * (p->nq + 2 * p->nkv));
    p->off_q = take(sizeof(float) * (size_t)B * p->n_q);
    p->off_kv_new = take(sizeof(float) * (size_t)B * 2 * p->nkv * p->D);
    p->off_attn_o = take(sizeof(float) * (size_t)B * p->nq * p->max_chunks * p->D);
    p->off_attn_ml = take(sizeof(float) * (size_t)B * p->nq * p->max_chunks * 2);
    p->off_a = take(sizeof(float) * (size_t)B * p->n_q);
    p->off_a16 = take(sizeof(uint16_t) * (size_t)B * p->n_q);
    p->off_seq_chunk = take(sizeof(int32_t) * 2 * (size_t)B);
    p->ws_bytes = off;

    const size_t e = (size_t)p->elem;
    p->bytes_hidden = e * p->B * p->H;
    p->bytes_norm = e * p->H;
    p->bytes_wqkv = e * (size_t)p->H * p->n_qkv;
    p->bytes_wo = e * (size_t)p->n_q * p->H;
    p->bytes_cache = e * (size_t)p->B * p->cap * p->nkv * p->D;
    p->bytes_pos = sizeof(int32_t) * p->B;
    p->bytes_out = e * p->B * p->H;
    p->bytes_dbg = sizeof(float) * p->B * p->H;
    return DAB_OK;
}

dab_status make_ffn_plan(const dab_ffn_config* cfg, FfnPlan* p) {
    if (!cfg || !p) return DAB_ERR_INVALID_ARG;
    *p = FfnPlan();
    const dab_ffn_config& c = *cfg;
    if (c.batch < 0 || c.hidden <= 0 || c.intermediate <= 0) return DAB_ERR_INVALID_ARG;
    if (c.dtype != DAB_F32 && c.dtype != DAB_BF16) return DAB_ERR_INVALID_ARG;
    if (!(c.eps >= 0.f) || !isfinite(c.eps)) return DAB_ERR_INVALID_ARG;
    if (c.hidden % 64 != 0 || c.intermediate % 64 != 0) return DAB_ERR_UNSUPPORTED;
    // each GEMV workgroup keeps one batch row of its input (H, or F for the
    // down projection) in LDS as fp32
    if ((size_t)c.hidden * sizeof(float) > (size_t)kPanelLds ||
        (size_t)c.intermediate * sizeof(float) > (size_t)kPanelLds || c.batch > 4096)
        return DAB_ERR_UNSUPPORTED;
    p->B = c.batch;
    p->H = c.hidden;
    p->F = c.intermediate;
    p->dtype = c.dtype;
    p->elem = c.dtype == DAB_BF16 ? 2 : 4;
    p->eps = c.eps;
    const int B = p->B > 0 ? p->B : 1;
    // bf16 batches of 8 or more: MFMA panels, 16 sequences per workgroup (the
    // VALU panel holds at most 4 and is bound by its arithmetic there).  The
    // gate/up panel is 16 rows of W_gate and the same 16 rows of W_up, one
    // MFMA tile each, so both sums of an output meet in one workgroup.
    p->mfma = p->dtype == DAB_BF16 && B >= 8;
    if (p->mfma) {
        // gate/up: 16 rows of W_gate (tile 0) and the same rows of W_up (tile 1)
        PanelPlan& g = p->gu;
        g.K = p->H;
        g.N = 2 * p->F;
        g.mfma = true;
        g.rows = 16;
        g.panels = p->F / 16;
        // H of 1024, 2048 or 4096 (the streamed panel): panels of T mixed tiles, each 8 features with
        // their gate rows at tile rows 0-7 and their up rows at 8-15, T the smallest of 1, 2, 4, 7, 8
        // that makes at most one panel per CU and divides F (8B layer, F 14336: 256 panels of 7 tiles,
        // one round, against 896 two-tile panels in three and a half)
        if (p->H == 1024 || p->H == 2048 || p->H == 4096) {
            const int cus = 256, mixed = p->F / 8;
            const int choices[5] = {1, 2, 4, 7, 8};
            int tiles = 0;
            for (int i = 0; i < 5 && tiles == 0; ++i)
                if (mixed % choices[i] == 0 && mixed / choices[i] <= cus) tiles = choices[i];
            for (int i = 4; i >= 0 && tiles == 0; --i)           // many features: the largest that divides
                if (mixed % choices[i] == 0) tiles = choices[i];
            if (tiles > 0 && p->F % 8 == 0) {
                p->gu_tiles = tiles;
                g.rows = 8 * tiles;
                g.panels = p->F / (8 * tiles);
            }
        }
        g.nb = B > 16 ? 32 : 16;
        g.nbg = ceil_div(B, g.nb);
        g.grid = g.nbg == 1 ? g.panels : (int)align_up((size_t)g.panels, 8) * g.nbg;
        if (!plan_mfma_panel(p->F, p->H, B, false, 0, &p->down)) return DAB_ERR_UNSUPPORTED;
    } else if (!plan_panel(p->H, 2 * p->F, B, 2, &p->gu) || !plan_panel(p->F, p->H, B, 2, &p->down)) {
        return DAB_ERR_UNSUPPORTED;
    }
    p->off_m = 0;
    p->off_m16 = align_up(sizeof(float) * (size_t)B * p->F, 256);
    p->off_hand = p->off_m16 + align_up(sizeof(uint16_t) * (size_t)B * p->F, 256);
    p->ws_bytes = p->off_hand + align_up(sizeof(int32_t) * (size_t)h_region(B), 256);
    const size_t e = (size_t)p->elem;
    p->bytes_hidden = e * p->B * p->H;
    p->bytes_norm = e * p->H;
    p->bytes_wgu = e * (size_t)p->F * p->H;
    p->bytes_wdown = e * (size_t)p->H * p->F;
    p->bytes_out = e * p->B * p->H;
    p->bytes_dbg = sizeof(float) * p->B * p->H;
    return DAB_OK;
}

dab_status check_ffn_call(const FfnPlan& p, const void* hidden, const void* norm_w, const void* w_gate,
                          const void* w_up, const void* w_down, const void* out, const float* dbg_y,
                          const void* workspace, size_t ws_bytes) {
    if (!workspace) return DAB_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DAB_ERR_INVALID_ARG;
    if (ws_bytes < p.ws_bytes) return DAB_ERR_WORKSPACE;
    if (p.B == 0) return DAB_OK;  // nothing is read or written
    const void* req[] = {hidden, norm_w, w_gate, w_up, w_down, out};
    for (const void* q : req)
        if (!q || !aligned(q, 16)) return DAB_ERR_INVALID_ARG;
    if (dbg_y && !aligned(dbg_y, 16)) return DAB_ERR_INVALID_ARG;
    struct Span { const void* p; size_t n; bool written; };
    const Span spans[] = {
        {hidden, p.bytes_hidden, false}, {norm_w, p.bytes_norm, false}, {w_gate, p.bytes_wgu, false},
        {w_up, p.bytes_wgu, false},      {w_down, p.bytes_wdown, false}, {out, p.bytes_out, true},
        {dbg_y, p.bytes_dbg, true},      {workspace, p.ws_bytes, true},
    };
    const int n = (int)(sizeof(spans) / sizeof(spans[0]));
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j)
            if ((spans[i].written || spans[j].written) &&
                overlaps(spans[i].p, spans[i].n, spans[j].p, spans[j].n))
                return DAB_ERR_INVALID_ARG;
    return DAB_OK;
}

dab_status check_call(const Plan& p, const void* hidden, const void* norm_w, const void* w_qkv,
                      const void* w_o, const void* k_cache, const void* v_cache, const int32_t* pos,
                      const void* out, const float* dbg_y, const void* workspace, size_t ws_bytes) {
    if (!workspace) return DAB_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return DAB_ERR_INVALID_ARG;
    if (ws_bytes < p.ws_bytes) return DAB_ERR_WORKSPACE;
    if (p.B == 0) return DAB_OK;  // nothing is read or written
    const void* req[] = {hidden, norm_w, w_qkv, w_o, k_cache, v_cache, out};
    for (const void* q : req)
        if (!q || !aligned(q, 16)) return DAB_ERR_INVALID_ARG;
    if (!pos || !aligned(pos, 4)) return DAB_ERR_INVALID_ARG;
    if (dbg_y && !aligned(dbg_y, 16)) return DAB_ERR_INVALID_ARG;

    struct Span { const void* p; size_t n; bool written; };
    const Span spans[] = {
        {hidden, p.bytes_hidden, false}, {norm_w, p.bytes_norm, false}, {w_qkv, p.bytes_wqkv, false},
        {w_o, p.bytes_wo, false},        {pos, p.bytes_pos, false},     {k_cache, p.bytes_cache, true},
        {v_cache, p.bytes_cache, true},  {out, p.bytes_out, true},      {dbg_y, p.bytes_dbg, true},
        {workspace, p.ws_bytes, true},
    };
    const int n = (int)(sizeof(spans) / sizeof(spans[0]));
    for (int i = 0; i < n; ++i)
        for (int j = i + 1; j < n; ++j)
            if ((spans[i].written || spans[j].written) &&
                overlaps(spans[i].p, spans[i].n, spans[j].p, spans[j].n))
                return DAB_ERR_INVALID_ARG;
    return DAB_OK;
}

dab_status check_layer_call(const Plan& p, const FfnPlan& f, const void* hidden, const void* attn_norm_w,
                            const void* w_qkv, const void* w_o, const void* k_cache, const void* v_cache,
                            const int32_t* pos, const void* ffn_norm_w, const void* w_gate, const void* w_up,
                            const void* w_down, const void* h, const void* out, const void* workspace,
                            size_t ws_bytes, const void* ffn_workspace, size_t ffn_ws_bytes) {
    if (f.B != p.B || f.H != p.H || f.dtype != p.dtype) return DAB_ERR_INVALID_ARG;
    dab_status st = check_call(p, hidden, attn_norm_w, w_qkv, w_o, k_cache, v_cache, pos, h, nullptr, workspace,
                               ws_bytes);
    if (st != DAB_OK) return st;
    st = check_ffn_call(f, h, ffn_norm_w, w_gate, w_up, w_down, out, nullptr, ffn_workspace, ffn_ws_bytes);
    if (st != DAB_OK) return st;
    if (p.B == 0) return DAB_OK;
    // across the halves: what one half writes overlaps nothing of the other
    struct Span { const void* p; size_t n; };
    const Span attn[] = {{hidden, p.bytes_hidden}, {attn_norm_w, p.bytes_norm}, {w_qkv, p.bytes_wqkv},
                         {w_o, p.bytes_wo},         {pos, p.bytes_pos},          {k_cache, p.bytes_cache},
                         {v_cache, p.bytes_cache},  {workspace, p.ws_bytes},   {h, p.bytes_out}};
    const Span ffn[] = {{ffn_norm_w, f.bytes_norm}, {w_gate, f.bytes_wgu}, {w_up, f.bytes_wgu},
                        {w_down, f.bytes_wdown},     {out, f.bytes_out},    {ffn_workspace, f.ws_bytes}};
    const int n_attn = (int)(sizeof(attn) / sizeof(attn[0])), n_ffn = (int)(sizeof(ffn) / sizeof(ffn[0]));
    for (int i = 0; i < n_attn; ++i)
        for (int j = 0; j < n_ffn; ++j) {
            // attention inputs read only (hidden, weights, pos) against FFN inputs read only
            const bool attn_written = i >= 5, ffn_written = j >= 4;
            if ((attn_written || ffn_written) && overlaps(attn[i].p, attn[i].n, ffn[j].p, ffn[j].n))
                return DAB_ERR_INVALID_ARG;
        }
    return DAB_OK;
}

}  // namespace dab
