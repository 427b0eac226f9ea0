// The C ABI (include/densegemm.h): argument checks, tile choice, launches.
#include <string.h>

#include <mutex>

#include "internal.hpp"

namespace dg {

hipError_t launch_tiled_rung(int kernel, int dt, int idx, const GemmArgs& a, hipStream_t s)
{
    const int mode = a.sk_count ? MODE_SK : a.splits > 1 ? MODE_SPLIT : (a.ep.on ? MODE_EPI : MODE_PLAIN);
    const int fam = kernel == GEMM_KERNEL_TILED ? 0 : 1;
#define DG_PICK(D, M, F) \
    if (dt == D && mode == M && fam == F) return launch_inst_##D##_##M##_##F(kernel, idx, a, s);
    DG_PICK(0, 0, 0) DG_PICK(0, 0, 1) DG_PICK(0, 1, 0) DG_PICK(0, 1, 1) DG_PICK(0, 2, 0)
    DG_PICK(0, 2, 1) DG_PICK(1, 0, 0) DG_PICK(1, 0, 1) DG_PICK(1, 1, 0) DG_PICK(1, 1, 1)
    DG_PICK(1, 2, 0) DG_PICK(1, 2, 1) DG_PICK(0, 3, 0) DG_PICK(0, 3, 1) DG_PICK(1, 3, 0)
    DG_PICK(1, 3, 1)
#undef DG_PICK
    return hipErrorInvalidValue;
}

SkPlan sk_plan(int kernel, int idx, int tm, int tn, int64_t M, int64_t N, int64_t K, int e, int grid)
{
    SkPlan pl;
    memset(&pl, 0, sizeof pl);
    if ((kernel != GEMM_KERNEL_TILED && kernel != GEMM_KERNEL_TILED_AB) || !sk_rung(tm, tn) ||
        M <= 0 || N <= 0 || K <= 0 || grid <= 0 || grid > GEMM_STREAM_K_MAX_GRID)
        return pl;
    const int kpk = rung_ktb(kernel, idx) / 64;   // 64-byte blocks per k-tile
    if (kpk <= 0)
        return pl;
    const int64_t kblocks = (K * e + 63) / 64;
    const int nkt = (int)((kblocks + kpk - 1) / kpk);
    const int64_t tiles = ((M + tm - 1) / tm) * ((N + tn - 1) / tn);
    // whole tiles: every full round but the last when there is a stray one
    const int64_t dp = tiles >= grid ? (tiles / grid - (tiles % grid ? 1 : 0)) * grid : 0;
    const int64_t units = (tiles - dp) * nkt;
    if (units != 0 && units < grid)
        return pl;                 // a workgroup would get no unit
    if (tiles > INT32_MAX || units > (INT64_C(1) << 40))
        return pl;
    pl.ok = true;
    pl.grid = grid;
    pl.dp_tiles = (int)dp;
    pl.nkt = nkt;
    pl.tiles = tiles;
    // partial slots for the largest grid, so the size does not depend on the
    // device; counters for every tile (an upper bound of the stream-K ones)
    pl.slot_bytes = (int64_t)GEMM_STREAM_K_MAX_GRID * 2 * tm * tn * 4;
    pl.ws_bytes = pl.slot_bytes + (tiles * 4 + 255) / 256 * 256;
    return pl;
}

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    int checked = 0;
    int gfx950 = 0;
    int cus = 0;
};

std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices];

// Current device: is it gfx950, and how many CUs.  Cached per device.
gemm_status device_info(int* cus)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return GEMM_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceInfo& d = g_dev[dev];
    if (!d.checked) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return GEMM_ERR_HIP;
        d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        d.cus = prop.multiProcessorCount;
        d.checked = 1;
    }
    if (!d.gfx950)
        return GEMM_ERR_UNSUPPORTED;
    *cus = d.cus;
    return GEMM_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kMaxKSplit = 64;

// Split-K plan of a resolved tile (S == 1: none).
SplitPlan tile_split(const gemm_tile& t, int idx, int64_t M, int64_t N, int64_t K, int e)
{
    if (t.kernel == GEMM_KERNEL_SKINNY || t.k_split <= 1 || K == 0)
        return SplitPlan{1, 0, 0, 0};
    return split_plan(M, N, K, e, rung_ktb(t.kernel, idx), t.k_split);
}

// The ladder rung a tile names, if it is usable for this shape: atom 0 means
// 16; tile_k (elements) and lds_stages 0 mean the first rung that matches
// the other fields.
bool resolve_tile(const gemm_tile& t, int64_t M, int e, int* idx)
{
    if (t.tile_k < 0 || t.tile_k > 4096 || t.lds_stages < 0 || t.k_split < 0 ||
        (t.kernel != GEMM_KERNEL_SKINNY && t.k_split > kMaxKSplit))
        return false;
    // stream-K: one-pass tiled / A+B rungs with a stream-K instance
    if (t.stream_k != 0 &&
        (t.stream_k != 1 || (t.kernel != GEMM_KERNEL_TILED && t.kernel != GEMM_KERNEL_TILED_AB) ||
         !sk_rung(t.tile_m, t.tile_n) || t.k_split > 1))
        return false;
    const int atom = t.atom == 0 ? 16 : t.atom;
    const int ktb = t.tile_k * e;
    *idx = -1;
    if (t.kernel == GEMM_KERNEL_TILED)
        *idx = tiled_rung(t.tile_m, t.tile_n, t.waves, atom, t.lds_stages, ktb);
    else if (t.kernel == GEMM_KERNEL_TILED_AB)
        *idx = ab_rung(t.tile_m, t.tile_n, t.waves, atom, t.lds_stages, ktb);
    if ((t.kernel == GEMM_KERNEL_TILED || t.kernel == GEMM_KERNEL_TILED_AB) && *idx >= 0 &&
        !atom_fits_rt(e == 2 ? DT_BF16 : DT_FP8, atom, rung_ktb(t.kernel, *idx)))
        *idx = -1;
    else if (t.kernel == GEMM_KERNEL_TILED_PP)
        *idx = pp_rung(t.tile_m, t.tile_n, t.waves, atom, t.lds_stages, ktb);
    else if (t.kernel == GEMM_KERNEL_SKINNY)
        *idx = skinny_supported(t.tile_m, t.tile_n, t.k_split == 0 ? 4 : t.k_split) && M <= t.tile_m
                   ? 0
                   : -1;
    return *idx >= 0;
}

// The epilogue's arguments, checked; false if any is invalid.
bool make_epilogue(const gemm_epilogue* e, int64_t N, Epilogue* out)
{
    memset(out, 0, sizeof *out);
    if (!e)
        return true;
    if (e->activation < GEMM_ACT_NONE || e->activation > GEMM_ACT_GELU_TANH)
        return false;
    if (((uintptr_t)e->bias & 1u) || ((uintptr_t)e->scale_m & 3u) ||
        ((uintptr_t)e->scale_n & 3u) || ((uintptr_t)e->mul & 1u))
        return false;
    if (e->mul && (e->ld_mul < N || e->ld_mul * 2 > (INT64_C(1) << 22)))
        return false;
    out->bias = e->bias;
    out->scale_m = e->scale_m;
    out->scale_n = e->scale_n;
    out->mul = e->mul;
    out->ldmul = e->mul ? e->ld_mul : 0;
    out->mul_vec = e->mul && ((uintptr_t)e->mul & 15u) == 0 && e->ld_mul % 8 == 0;
    out->act = e->activation;
    out->on = e->bias || e->scale_m || e->scale_n || e->mul || e->activation != GEMM_ACT_NONE;
    return true;
}

// One GEMM launch (and its split-K reduction) of a resolved tile.
hipError_t launch_gemm(int dt, const gemm_tile& t, int idx, const SplitPlan& pl, const void* A,
                       int64_t lda, const void* Bs, const float* sa, const float* sb, uint16_t* C,
                       int64_t ldc, int64_t M, int64_t N, int64_t K, const Epilogue& ep, void* ws,
                       hipStream_t s, const SkPlan* sk = nullptr)
{
    const int e = dt == DT_BF16 ? 2 : 1;
    GemmArgs a;
    memset(&a, 0, sizeof a);
    a.A = static_cast<const uint8_t*>(A);
    a.Bs = static_cast<const uint8_t*>(Bs);
    a.C = C;
    a.sa = sa;
    a.sb = sb;
    a.lda_b = lda * e;
    a.ldc = ldc;
    a.M = (int)M;
    a.N = (int)N;
    a.KA_b = (int)(K * e);
    a.KB = (int)((K * e + 63) / 64);
    a.nkt = (a.KB + 1) / 2;
    a.tail = (a.KA_b % 128) != 0;
    a.nblk = (int)((N + 15) / 16);
    a.c_vec = (((uintptr_t)C & 15u) == 0) && (ldc % 8 == 0);
    a.splits = pl.S;
    a.kt_per = pl.kt_per;
    a.ldw = pl.ldw;
    a.ws = pl.S > 1 ? static_cast<float*>(ws) : nullptr;
    a.ep = ep;
    if (t.kernel == GEMM_KERNEL_SKINNY)
        return launch_skinny(dt, t.tile_m, t.tile_n, t.k_split == 0 ? 4 : t.k_split, a, s);
    a.tiles_m = (int)((M + t.tile_m - 1) / t.tile_m);
    a.tiles_n = (int)((N + t.tile_n - 1) / t.tile_n);
    if (t.stream_k && sk && sk->ok) {
        a.splits = sk->grid;             // the persistent grid
        a.sk_dp_tiles = sk->dp_tiles;
        a.sk_nkt = sk->nkt;
        a.ws = static_cast<float*>(ws);
        a.sk_count = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(ws) + sk->slot_bytes);
        hipError_t err = launch_zero_u32(a.sk_count, (int)(sk->tiles - sk->dp_tiles), s);
        if (err == hipSuccess)
            err = launch_tiled_rung(t.kernel, dt, idx, a, s);
        return err;
    }
    hipError_t err = launch_tiled_rung(t.kernel, dt, idx, a, s);
    if (err == hipSuccess && pl.S > 1)
        err = launch_splitk_reduce(a.ws, pl.S, a.M, a.N, pl.ldw, C, ldc, sa, sb, ep, s);
    return err;
}

// Columns of the first of two launches when the chosen one-pass tiled tile
// would run a last round of tiles that fills at most a quarter of the CUs
// after two or more full rounds (0: one launch).  The first launch takes the
// columns whose tiles fill the full rounds exactly or nearly; the second the
// rest.
int64_t tail_split_columns(const gemm_tile& t, const SplitPlan& pl, int64_t M, int64_t N, int cus)
{
    if (t.kernel == GEMM_KERNEL_SKINNY || pl.S > 1 || cus <= 0)
        return 0;
    const int64_t tiles_m = (M + t.tile_m - 1) / t.tile_m;
    const int64_t tiles_n = (N + t.tile_n - 1) / t.tile_n;
    const int64_t tiles = tiles_m * tiles_n;
    const int64_t full = tiles / cus, left = tiles % cus;
    if (full < 2 || left == 0 || 4 * left > cus)
        return 0;
    const int64_t n_main = full * cus / tiles_m * t.tile_n;
    return n_main > 0 && n_main < N ? n_main : 0;
}

// The launches of a GEMM whose tile the library chooses: one tile for all
// N columns, or, when the chosen one-pass tile would leave a last round of
// tiles that fills at most a quarter of the CUs (tail_split_columns), the
// columns that fill whole rounds with it and the rest as a second GEMM with a
// tile chosen for that narrower shape -- if that second GEMM costs less than
// the stray round.  Measured on MI355X: the stray round costs about 40 % of a
// round (its tiles start while the last full round drains), and a small GEMM
// at least about 6 us (launch, cold prologue, epilogue), more than the model
// gives it.  Or, when no column split applies, the rows whose tiles of a
// large rung fill whole rounds and the rest as a second GEMM (row_split).
// False if a chosen tile names no rung (never, for the selector's own
// choices).
struct AutoPlan {
    gemm_tile t1, t2;
    int idx1, idx2;
    SplitPlan pl1, pl2;
    SkPlan sk1;    // the first launch's stream-K plan when t1.stream_k
    int64_t n1;    // columns of the first launch; N: all of them
    int64_t m1;    // rows of the first launch; M: all of them (at most one of
                   // n1, m1 splits)
};

// Row split.  A shape whose tiles make one or more whole rounds plus a
// stray part (GPT-3-XL dX, 10240 x 2048 x 8192: 320 tiles of 256 x 256 on
// 256 CUs) runs the rows [0, m1) that fill whole rounds with a large tile
// and the remaining rows as a second GEMM with a tile of their own, when the
// model prices the pair, plus 3 us for the second launch starting only once
// the first has drained, below 95 % of the single launch.  Candidates are the
// 256 x 256, 256 x 128 and 128 x 256 tiles whose column count divides the
// CUs, so that m1 rows make whole rounds; the first launch must choose that
// tile for its rows.  The column split takes precedence.  Measured on
// MI355X (graph replay, single launch -> two): 10240 x 2048 x 8192
// 301.6 -> 269.2-270.4 us, 10240 x 2048 x 2048 88.0 -> 80.8, 8704 x 2048 x
// 1024 44.9 -> 42.7, 8448 x 1024 x 2048 50.2 -> 47.3, 9216 x 2048 x 1024
// 45.9 -> 44.0; without the 3 us, 8704 x 2048 x 512 was also split and
// went 27.6 -> 29.3 (its launches are short), and 9216 x 1024 x 2048 gained
// 1 %, which the rule now leaves as one launch.
bool row_split(int64_t M, int64_t N, int64_t K, int dt, int cus, size_t ws_bytes, AutoPlan* ap)
{
    const int e = dt == DT_BF16 ? 2 : 1;
    constexpr double kMinGemmUs = 6.0, kSecondLaunchUs = 3.0;
    constexpr int kShapes[3][2] = {{256, 256}, {256, 128}, {128, 256}};
    double best = 0.95 * (double)ap->t1.predicted_us;
    bool found = false;
    AutoPlan cand = *ap;
    for (const auto& sh : kShapes) {
        const int tm = sh[0], tn = sh[1];
        const int64_t tiles_n = (N + tn - 1) / tn;
        if (tiles_n > cus || cus % tiles_n != 0)
            continue;
        const int64_t rows_round = (int64_t)(cus / tiles_n) * tm;
        const int64_t m1 = M / rows_round * rows_round;
        if (m1 == 0 || m1 >= M)
            continue;
        gemm_tile ta, tb;
        int ia = -1, ib = -1;
        choose_tile(m1, N, K, dt, cus, ws_bytes, &ta);
        if (ta.kernel == GEMM_KERNEL_SKINNY || ta.tile_m != tm || ta.tile_n != tn ||
            ta.k_split > 1 || !resolve_tile(ta, m1, e, &ia))
            continue;
        choose_tile(M - m1, N, K, dt, cus, ws_bytes, &tb);
        if (!resolve_tile(tb, M - m1, e, &ib))
            continue;
        const SplitPlan pa = tile_split(ta, ia, m1, N, K, e);
        const SplitPlan pb = tile_split(tb, ib, M - m1, N, K, e);
        if (pa.ws_bytes > (int64_t)ws_bytes || pb.ws_bytes > (int64_t)ws_bytes)
            continue;
        const double price =
            (double)ta.predicted_us + std::max((double)tb.predicted_us, kMinGemmUs) + kSecondLaunchUs;
        if (price < best) {
            best = price;
            found = true;
            cand.t1 = ta;
            cand.idx1 = ia;
            cand.pl1 = pa;
            cand.t2 = tb;
            cand.idx2 = ib;
            cand.pl2 = pb;
            cand.m1 = m1;
        }
    }
    if (found) {
        memset(&cand.sk1, 0, sizeof cand.sk1);
        *ap = cand;
    }
    return found;
}

// Stream-K in place of a one-pass tile that fills less than one round of
// the CUs, priced from measurements on MI355X (LLaMA prefill 597 x 11008 x
// 4096 on 128 x 256 tiles, per-phase timestamps): a k-tile unit takes about
// 1.45 times as long as in the one-pass launch (every CU streams, and
// neighbouring workgroups read different K ranges of the same tiles, so the
// L2 serves fewer re-reads), and a cut tile's fix-up (partials written
// through to memory, read back past the caches) costs about 20 us at the
// end of the launch.  Taken when that is below 95 % of the one-pass time:
// shapes whose tiles leave most CUs idle.
constexpr double kSkUnitSlowdown = 1.45;
constexpr double kSkFixupUs = 20.0;

bool plan_auto(int64_t M, int64_t N, int64_t K, int dt, int cus, size_t ws_bytes, AutoPlan* ap,
               bool allow_sk = true)
{
    const int e = dt == DT_BF16 ? 2 : 1;
    memset(ap, 0, sizeof *ap);
    ap->n1 = N;
    ap->m1 = M;
    choose_tile(M, N, K, dt, cus, ws_bytes, &ap->t1);
    if (!resolve_tile(ap->t1, M, e, &ap->idx1))
        return false;
    ap->pl1 = tile_split(ap->t1, ap->idx1, M, N, K, e);
    if (ap->pl1.ws_bytes > (int64_t)ws_bytes)
        return false;
    if (allow_sk && ap->pl1.S == 1 && ap->t1.kernel != GEMM_KERNEL_SKINNY) {
        const int grid = std::min(cus, (int)GEMM_STREAM_K_MAX_GRID);
        const SkPlan sk = sk_plan(ap->t1.kernel, ap->idx1, ap->t1.tile_m, ap->t1.tile_n, M, N, K,
                                  e, grid);
        if (sk.ok && sk.tiles < grid && sk.ws_bytes <= (int64_t)ws_bytes) {
            const double t_sk =
                ap->t1.predicted_us * kSkUnitSlowdown * (double)sk.tiles / grid + kSkFixupUs;
            if (t_sk < 0.95 * ap->t1.predicted_us) {
                ap->t1.stream_k = 1;
                ap->t1.predicted_us = (float)t_sk;
                ap->sk1 = sk;
                return true;
            }
        }
    }
    const int64_t n1 = tail_split_columns(ap->t1, ap->pl1, M, N, cus);
    if (n1 != 0) {
        gemm_tile t2;
        int idx2 = -1;
        choose_tile(M, N - n1, K, dt, cus, ws_bytes, &t2);
        const int64_t tiles = ((M + ap->t1.tile_m - 1) / ap->t1.tile_m) *
                              ((N + ap->t1.tile_n - 1) / ap->t1.tile_n);
        const double round_us = ap->t1.predicted_us / (double)((tiles + cus - 1) / cus);
        constexpr double kMinGemmUs = 6.0;
        if (resolve_tile(t2, M, e, &idx2) &&
            std::max((double)t2.predicted_us, kMinGemmUs) < 0.4 * round_us) {
            const SplitPlan pl2 = tile_split(t2, idx2, M, N - n1, K, e);
            if (pl2.ws_bytes <= (int64_t)ws_bytes) {
                ap->t2 = t2;
                ap->idx2 = idx2;
                ap->pl2 = pl2;
                ap->n1 = n1;
                return true;
            }
        }
    }
    if (ap->t1.kernel != GEMM_KERNEL_SKINNY)
        row_split(M, N, K, dt, cus, ws_bytes, ap);
    return true;
}

gemm_status run_gemm(int dt, const void* A, int64_t lda, const void* Bs, const float* sa,
                     const float* sb, uint16_t* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                     const gemm_tile* tile, const gemm_epilogue* epi, void* ws, size_t ws_bytes,
                     void* stream)
{
    const int e = dt == DT_BF16 ? 2 : 1;
    // ---- argument checks (no HIP call before this block ends)
    if (M < 0 || N < 0 || K < 0)
        return GEMM_ERR_INVALID_VALUE;
    if (M == 0 || N == 0)
        return GEMM_OK;
    // With K == 0 neither A, Bs nor the scales are read (empty sum).
    if (!C || (K > 0 && (!A || !Bs || (dt == DT_FP8 && (!sa || !sb)))))
        return GEMM_ERR_INVALID_VALUE;
    if (lda < K || ldc < N)
        return GEMM_ERR_INVALID_VALUE;
    if ((K > 0 && (!aligned16(A) || !aligned16(Bs) || (lda * e) % 16 != 0)) ||
        ((uintptr_t)C & 1u) != 0)
        return GEMM_ERR_INVALID_VALUE;
    if (ws_bytes > 0 && (!ws || !aligned16(ws)))
        return GEMM_ERR_INVALID_VALUE;
    Epilogue ep;
    if (!make_epilogue(epi, N, &ep))
        return GEMM_ERR_INVALID_VALUE;
    if (K % (dt == DT_BF16 ? 16 : 64) != 0)
        return GEMM_ERR_UNSUPPORTED;
    // 32-bit buffer offsets: a tile of up to 256 rows of A or C, and one
    // 16-column block of Bs, must stay below 2^31 bytes.
    if (M > INT32_MAX || N > INT32_MAX || lda * e > (INT64_C(1) << 22) ||
        ldc * 2 > (INT64_C(1) << 22) || K * e > (INT64_C(1) << 20))
        return GEMM_ERR_UNSUPPORTED;
    gemm_tile t;
    int idx = -1;
    SplitPlan pl{1, 0, 0, 0};
    SkPlan sk;
    memset(&sk, 0, sizeof sk);
    if (tile) {
        t = *tile;
        if (!resolve_tile(t, M, e, &idx))
            return GEMM_ERR_UNSUPPORTED;
        if (t.stream_k) {
            // no fused epilogue with stream-K; the workspace is checked with
            // the largest grid, the launch uses the device's
            if (ep.on || t.k_split > 1)
                return GEMM_ERR_UNSUPPORTED;
            const SkPlan chk = sk_plan(t.kernel, idx, t.tile_m, t.tile_n, M, N, K, e,
                                       GEMM_STREAM_K_MAX_GRID);
            if (!chk.ok)
                return GEMM_ERR_UNSUPPORTED;
            if (chk.ws_bytes > (int64_t)ws_bytes)
                return ws_bytes == 0 ? GEMM_ERR_UNSUPPORTED : GEMM_ERR_INVALID_VALUE;
        }
        pl = tile_split(t, idx, M, N, K, e);
        if (pl.S > 1 && !partial_plane_fits(M, pl.ldw))
            return GEMM_ERR_UNSUPPORTED;
        if (pl.ws_bytes > (int64_t)ws_bytes)
            return ws_bytes == 0 ? GEMM_ERR_UNSUPPORTED : GEMM_ERR_INVALID_VALUE;
    }
    // ---- device
    int cus = 0;
    gemm_status st = device_info(&cus);
    if (st != GEMM_OK)
        return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (K == 0)
        return launch_zero_c(C, ldc, M, N, ep, s) == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
    if (tile && t.stream_k) {
        sk = sk_plan(t.kernel, idx, t.tile_m, t.tile_n, M, N, K, e,
                     std::min(cus, (int)GEMM_STREAM_K_MAX_GRID));
        if (!sk.ok)
            return GEMM_ERR_UNSUPPORTED;
    }
    if (!tile) {
        AutoPlan ap;
        if (!plan_auto(M, N, K, dt, cus, ws_bytes, &ap, !ep.on))
            return GEMM_ERR_UNSUPPORTED;   // the selector names only rungs that exist
        t = ap.t1;
        idx = ap.idx1;
        pl = ap.pl1;
        sk = ap.sk1;
        // The fused-epilogue instance of the 4-wave e4m3 256 x 256 rung (the
        // whole-line-A kernel) spills 3 VGPRs: with per-row and per-column
        // scales on 4096^3 it measured 66-69 us on MI355X against 58-60 us for
        // the 8-wave rung of the same tile (54-61 us for both without an
        // epilogue).  A fused launch that the selector puts on it takes the
        // 8-wave rung.  (Calibrated rung costs are for plain launches.)
        if (ep.on && dt == DT_FP8 && ap.n1 == N && ap.m1 == M && t.kernel == GEMM_KERNEL_TILED_AB &&
            t.tile_m == 256 && t.tile_n == 256 && t.waves == 4 && t.atom == 32 &&
            t.lds_stages == 4 && t.tile_k == 64 && t.k_split <= 1) {
            gemm_tile t8 = t;
            t8.waves = 8;
            int idx8 = -1;
            if (resolve_tile(t8, M, e, &idx8)) {
                t = t8;
                idx = idx8;
                pl = tile_split(t, idx, M, N, K, e);
            }
        }
        if (ap.n1 < N) {
            const int64_t n1 = ap.n1;
            const int64_t be = 64 * ((K * e + 63) / 64) * 16;   // Bs bytes per 16 columns
            Epilogue ep2 = ep;
            if (ep2.bias)
                ep2.bias += n1;
            if (ep2.scale_n)
                ep2.scale_n += n1;
            if (ep2.mul) {
                ep2.mul += n1;
                ep2.mul_vec = ((uintptr_t)ep2.mul & 15u) == 0 && ep2.ldmul % 8 == 0;
            }
            hipError_t err =
                launch_gemm(dt, t, idx, pl, A, lda, Bs, sa, sb, C, ldc, M, n1, K, ep, ws, s);
            if (err == hipSuccess)
                err = launch_gemm(dt, ap.t2, ap.idx2, ap.pl2, A, lda,
                                  static_cast<const uint8_t*>(Bs) + n1 / 16 * be, sa, sb, C + n1,
                                  ldc, M, N - n1, K, ep2, ws, s);
            return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
        }
        if (ap.m1 < M) {
            const int64_t m1 = ap.m1;
            Epilogue ep2 = ep;
            if (ep2.scale_m)
                ep2.scale_m += m1;
            if (ep2.mul) {
                ep2.mul += m1 * ep2.ldmul;
                ep2.mul_vec = ((uintptr_t)ep2.mul & 15u) == 0 && ep2.ldmul % 8 == 0;
            }
            hipError_t err =
                launch_gemm(dt, t, idx, pl, A, lda, Bs, sa, sb, C, ldc, m1, N, K, ep, ws, s);
            if (err == hipSuccess)
                err = launch_gemm(dt, ap.t2, ap.idx2, ap.pl2,
                                  static_cast<const uint8_t*>(A) + m1 * lda * e, lda, Bs, sa, sb,
                                  C + m1 * ldc, ldc, M - m1, N, K, ep2, ws, s);
            return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
        }
    }
    const hipError_t err =
        launch_gemm(dt, t, idx, pl, A, lda, Bs, sa, sb, C, ldc, M, N, K, ep, ws, s, &sk);
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

// ---- scratch for callers that cannot allocate (gemm_bf16_noalloc)
//
// The split-K partials of gemm_bf16_noalloc live in this file-scope device
// array: each GPU the library runs on holds its own copy, at its own
// address, until the process ends.  In host code `scratch` is a host-side
// stand-in, not a device address; the device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// pointer is handed to kernels.
static __device__ __align__(256) uint8_t scratch[GEMM_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];

// The current device's copy of `scratch`: its device address, looked up on
// the first call on that device.  NULL if the lookup fails.
void* device_scratch()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return nullptr;
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

}  // namespace
}  // namespace dg

extern "C" {

gemm_status gemm_bf16_noalloc(const uint16_t* A, int64_t lda, const void* Bs, uint16_t* C,
                              int64_t ldc, int64_t M, int64_t N, int64_t K, const gemm_tile* tile,
                              void* stream)
{
    // A forced split-K tile whose partials exceed the scratch array is
    // refused before any device call.
    if (tile && M > 0 && N > 0 && K > 0 &&
        gemm_workspace_bytes(M, N, K, GEMM_BF16, tile) > (size_t)GEMM_NOALLOC_SCRATCH_BYTES)
        return GEMM_ERR_INVALID_VALUE;
    void* ws = dg::device_scratch();
    if (!ws)
        return GEMM_ERR_HIP;
    return dg::run_gemm(dg::DT_BF16, A, lda, Bs, nullptr, nullptr, C, ldc, M, N, K, tile, nullptr,
                        ws, (size_t)GEMM_NOALLOC_SCRATCH_BYTES, stream);
}

gemm_status gemm_bf16(const uint16_t* A, int64_t lda, const void* Bs, uint16_t* C, int64_t ldc,
                      int64_t M, int64_t N, int64_t K, const gemm_tile* tile, void* stream)
{
    return dg::run_gemm(dg::DT_BF16, A, lda, Bs, nullptr, nullptr, C, ldc, M, N, K, tile, nullptr,
                        nullptr, 0, stream);
}

gemm_status gemm_fp8_scaled(const uint8_t* A, int64_t lda, const void* Bs, const float* scale_a,
                            const float* scale_b, uint16_t* C, int64_t ldc, int64_t M, int64_t N,
                            int64_t K, const gemm_tile* tile, void* stream)
{
    return dg::run_gemm(dg::DT_FP8, A, lda, Bs, scale_a, scale_b, C, ldc, M, N, K, tile, nullptr,
                        nullptr, 0, stream);
}

gemm_status gemm_bf16_ws(const uint16_t* A, int64_t lda, const void* Bs, uint16_t* C, int64_t ldc,
                         int64_t M, int64_t N, int64_t K, const gemm_tile* tile, void* workspace,
                         size_t workspace_bytes, void* stream)
{
    return dg::run_gemm(dg::DT_BF16, A, lda, Bs, nullptr, nullptr, C, ldc, M, N, K, tile, nullptr,
                        workspace, workspace_bytes, stream);
}

gemm_status gemm_fp8_scaled_ws(const uint8_t* A, int64_t lda, const void* Bs,
                               const float* scale_a, const float* scale_b, uint16_t* C,
                               int64_t ldc, int64_t M, int64_t N, int64_t K,
                               const gemm_tile* tile, void* workspace, size_t workspace_bytes,
                               void* stream)
{
    return dg::run_gemm(dg::DT_FP8, A, lda, Bs, scale_a, scale_b, C, ldc, M, N, K, tile, nullptr,
                        workspace, workspace_bytes, stream);
}

gemm_status gemm_bf16_ex(const uint16_t* A, int64_t lda, const void* Bs, uint16_t* C, int64_t ldc,
                         int64_t M, int64_t N, int64_t K, const gemm_tile* tile,
                         const gemm_epilogue* epilogue, void* workspace, size_t workspace_bytes,
                         void* stream)
{
    return dg::run_gemm(dg::DT_BF16, A, lda, Bs, nullptr, nullptr, C, ldc, M, N, K, tile, epilogue,
                        workspace, workspace_bytes, stream);
}

gemm_status gemm_fp8_scaled_ex(const uint8_t* A, int64_t lda, const void* Bs,
                               const float* scale_a, const float* scale_b, uint16_t* C,
                               int64_t ldc, int64_t M, int64_t N, int64_t K,
                               const gemm_tile* tile, const gemm_epilogue* epilogue,
                               void* workspace, size_t workspace_bytes, void* stream)
{
    return dg::run_gemm(dg::DT_FP8, A, lda, Bs, scale_a, scale_b, C, ldc, M, N, K, tile, epilogue,
                        workspace, workspace_bytes, stream);
}

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, gemm_dtype dtype,
                            const gemm_tile* tile)
{
    if (!tile || M <= 0 || N <= 0 || K <= 0 || (dtype != GEMM_BF16 && dtype != GEMM_FP8_E4M3))
        return 0;
    const int e = dtype == GEMM_BF16 ? 2 : 1;
    int idx = -1;
    if (!dg::resolve_tile(*tile, M, e, &idx))
        return 0;
    if (tile->stream_k) {
        if (tile->k_split > 1)
            return 0;
        const dg::SkPlan sk = dg::sk_plan(tile->kernel, idx, tile->tile_m, tile->tile_n, M, N, K, e,
                                          GEMM_STREAM_K_MAX_GRID);
        return sk.ok ? (size_t)sk.ws_bytes : 0;
    }
    return (size_t)dg::tile_split(*tile, idx, M, N, K, e).ws_bytes;
}

size_t shuffle_b_bytes(int64_t N, int64_t K, gemm_dtype dtype)
{
    if (N < 0 || K < 0 || (dtype != GEMM_BF16 && dtype != GEMM_FP8_E4M3))
        return 0;
    const int64_t e = dtype == GEMM_BF16 ? 2 : 1;
    const int64_t kblocks = (K * e + 63) / 64;
    return (size_t)((N + 15) / 16 * 16 * kblocks * 64);
}

gemm_status shuffle_b(const void* B, int64_t ldb, void* Bs, int64_t N, int64_t K, gemm_dtype dtype,
                      void* stream)
{
    if (N < 0 || K < 0 || (dtype != GEMM_BF16 && dtype != GEMM_FP8_E4M3))
        return GEMM_ERR_INVALID_VALUE;
    if (N == 0 || K == 0)
        return GEMM_OK;
    if (!B || !Bs || ldb < K || !dg::aligned16(Bs))
        return GEMM_ERR_INVALID_VALUE;
    const int64_t e = dtype == GEMM_BF16 ? 2 : 1;
    if (K % (dtype == GEMM_BF16 ? 16 : 64) != 0)
        return GEMM_ERR_UNSUPPORTED;
    int cus = 0;
    gemm_status st = dg::device_info(&cus);
    if (st != GEMM_OK)
        return st;
    const int aligned = dg::aligned16(B) && (ldb * e) % 16 == 0;
    hipError_t err = dg::launch_shuffle_b(static_cast<const uint8_t*>(B), ldb * e,
                                          static_cast<uint8_t*>(Bs), N, K * e, (K * e + 63) / 64,
                                          aligned, reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

gemm_status gemm_read_probe(const void* buf, uint64_t bytes, uint32_t* out, void* stream)
{
    if (!buf || !out || bytes == 0 || bytes % 16 != 0 || bytes > (1ull << 40) || !dg::aligned16(buf))
        return GEMM_ERR_INVALID_VALUE;
    int cus = 0;
    gemm_status st = dg::device_info(&cus);
    if (st != GEMM_OK)
        return st;
    const hipError_t err = dg::launch_read_probe(buf, (int64_t)bytes, out, GEMM_READ_PROBE_SLOTS / 16,
                                                 reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

gemm_status shuffle_b_t(const void* Bt, int64_t ldbt, void* Bs, int64_t N, int64_t K,
                        gemm_dtype dtype, void* stream)
{
    if (N < 0 || K < 0 || (dtype != GEMM_BF16 && dtype != GEMM_FP8_E4M3))
        return GEMM_ERR_INVALID_VALUE;
    if (N == 0 || K == 0)
        return GEMM_OK;
    const int64_t e = dtype == GEMM_BF16 ? 2 : 1;
    if (!Bt || !Bs || ldbt < N || !dg::aligned16(Bs) || ((uintptr_t)Bt % e) != 0)
        return GEMM_ERR_INVALID_VALUE;
    if (K % (dtype == GEMM_BF16 ? 16 : 64) != 0)
        return GEMM_ERR_UNSUPPORTED;
    if (((K * e + 63) / 64 * 64 / e + 63) / 64 > 65535)    // k tiles: the grid's second axis
        return GEMM_ERR_UNSUPPORTED;
    int cus = 0;
    gemm_status st = dg::device_info(&cus);
    if (st != GEMM_OK)
        return st;
    hipError_t err = dg::launch_shuffle_bt(Bt, ldbt, static_cast<uint8_t*>(Bs), N, K, (int)e,
                                           reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

gemm_status transpose_2d(const void* src, int64_t ld_src, void* dst, int64_t ld_dst, int64_t rows,
                         int64_t cols, int32_t elem_bytes, void* stream)
{
    if (rows < 0 || cols < 0 || (elem_bytes != 1 && elem_bytes != 2))
        return GEMM_ERR_INVALID_VALUE;
    if (rows == 0 || cols == 0)
        return GEMM_OK;
    if (!src || !dst || ld_src < cols || ld_dst < rows || ((uintptr_t)src % elem_bytes) != 0 ||
        ((uintptr_t)dst % elem_bytes) != 0)
        return GEMM_ERR_INVALID_VALUE;
    if ((rows + 63) / 64 > 65535 || (cols + 63) / 64 > INT32_MAX)
        return GEMM_ERR_UNSUPPORTED;
    int cus = 0;
    gemm_status st = dg::device_info(&cus);
    if (st != GEMM_OK)
        return st;
    hipError_t err = dg::launch_transpose(src, ld_src, dst, ld_dst, rows, cols, elem_bytes,
                                          reinterpret_cast<hipStream_t>(stream));
    return err == hipSuccess ? GEMM_OK : GEMM_ERR_HIP;
}

gemm_status gemm_plan(int64_t M, int64_t N, int64_t K, gemm_dtype dtype, int32_t num_cus,
                      size_t workspace_bytes, gemm_tile* first, gemm_tile* second,
                      int64_t* first_columns, int64_t* first_rows)
{
    if (!first || !second || !first_columns || !first_rows || M <= 0 || N <= 0 || K <= 0 ||
        num_cus <= 0 ||
        (dtype != GEMM_BF16 && dtype != GEMM_FP8_E4M3))
        return GEMM_ERR_INVALID_VALUE;
    dg::AutoPlan ap;
    if (!dg::plan_auto(M, N, K, (int)dtype, num_cus, workspace_bytes, &ap))
        return GEMM_ERR_UNSUPPORTED;
    *first = ap.t1;
    *second = ap.t2;
    *first_columns = ap.n1;
    *first_rows = ap.m1;
    return GEMM_OK;
}

gemm_status gemm_tile_check(const gemm_tile* tile, int64_t M, gemm_dtype dtype)
{
    if (!tile || M < 0 || (dtype != GEMM_BF16 && dtype != GEMM_FP8_E4M3))
        return GEMM_ERR_INVALID_VALUE;
    int idx = -1;
    return dg::resolve_tile(*tile, M, dtype == GEMM_BF16 ? 2 : 1, &idx) ? GEMM_OK
                                                                        : GEMM_ERR_UNSUPPORTED;
}

const char* gemm_status_string(gemm_status status)
{
    switch (status) {
    case GEMM_OK:
        return "GEMM_OK";
    case GEMM_ERR_INVALID_VALUE:
        return "GEMM_ERR_INVALID_VALUE";
    case GEMM_ERR_UNSUPPORTED:
        return "GEMM_ERR_UNSUPPORTED";
    case GEMM_ERR_HIP:
        return "GEMM_ERR_HIP";
    }
    return "GEMM_ERR_UNKNOWN";
}

}  // extern "C"
