// select_tile: analytic choice of kernel and tile for an M x N x K GEMM.
//
// The model (pure host, deterministic).  Rungs measured on MI355X are priced
// by their calibrated cost (calibration.inc, fitted by calibrate.py from tile
// sweeps); the analytic model below prices the rest:
//   - tile quantization tile_eff = M*N / (M_pad*N_pad) and wave quantization
//     wq_eff = tiles / (rounds * slots) as the TraceLens GEMM analysis page
//     defines them ("Tile quantization efficiency", "Wave quantization
//     efficiency"); the padding screen of the FlyDSL PR #1303 page rejects a
//     tile whose padded output exceeds 1.25x the real one unless no other
//     tile is feasible;
//   - per-k-tile cost of a tiled workgroup = the largest of its MFMA issue
//     time, its LDS traffic and its global-load traffic ("GEMM Optimization
//     Guide" page, sections 1.5, 2.4, 8.3, 9.3), occupancy from the combined
//     VGPR budget of section 10.2, LDS budget of 160 KiB per CU;
//   - skinny (small M) candidates are priced as a stream of B at the HBM
//     rate, derated when fewer workgroups than CUs are in flight;
//   - the result is the candidate with the lowest predicted time; ties go to
//     the earlier candidate in a fixed order.
#include <math.h>
#include <string.h>

#include <mutex>
#include <unordered_map>

#include "internal.hpp"

namespace dg {

namespace {

// Measured per-rung cost constants (calibrate.py): t_us = a * n_cu * K_bytes
// / 1000 + b * n_cu + g * MB + c, n_cu = ceil(tiles / CUs), MB = bytes of A,
// B and C / 1e6.
struct RungCalib {
    int dt, kernel, tm, tn, waves, atom, st, ktb;
    float a, b, g, c;       // one-pass runs
    float as, bs, gs, cs;   // split-K runs: fitted jointly with the split costs
    int points;
};
// split-K costs beyond a rung's own time (calibrate.py)
struct SplitCalib {
    float d, r1, r0;
    int points;
};
// skinny rungs: t_us = a * per_cu * MB per workgroup + b * MB in total + c
struct SkinnyCalib {
    int dt, tm, tn, waves;
    float a, b, c;
    int points;
};
// the fastest tile measured on a swept shape
struct MeasuredBest {
    int dt;
    int64_t M, N, K;
    int kernel, tm, tn, tile_k, atom, waves, k_split, stages;
    float us;
};
#include "calibration.inc"

const RungCalib* find_calib(int dt, int kernel, int tm, int tn, int waves, int atom, int st,
                            int ktb)
{
    for (const RungCalib& r : kRungCalib)
        if (r.dt == dt && r.kernel == kernel && r.tm == tm && r.tn == tn && r.waves == waves &&
            r.atom == atom && r.st == st && r.ktb == ktb)
            return &r;
    return nullptr;
}

// Calibrated time of a tiled / A+B rung, or `fallback` if it was never
// measured.  With split-K, K is one slice's K and every tile counts `split`
// times.
double calibrated_us(int dt, int kernel, int tm, int tn, int waves, int atom, int st, int ktb,
                     int64_t M, int64_t N, int64_t K, int cus, double fallback, int split = 1)
{
    const RungCalib* r = find_calib(dt, kernel, tm, tn, waves, atom, st, ktb);
    if (!r)
        return fallback;
    const int e = dt == GEMM_BF16 ? 2 : 1;
    const int64_t tiles = ((M + tm - 1) / tm) * ((N + tn - 1) / tn) * split;
    const double ncu = (double)((tiles + cus - 1) / cus);
    // A, B and C bytes of the whole GEMM (K here is one slice's K)
    const double mb = ((double)M * K * e * split + (double)N * K * e * split + 2.0 * M * N) / 1e6;
    if (split > 1)
        return r->as * ncu * (double)K * e / 1000.0 + r->bs * ncu + r->gs * mb + r->cs;
    return r->a * ncu * (double)K * e / 1000.0 + r->b * ncu + r->g * mb + r->c;
}

struct Chip {
    double clock_hz = 2.4e9;
    double mfma_flop_per_clk_cu[2] = {4096.0, 8192.0};  // bf16, e4m3 dense
    double lds_bytes_per_clk = 128.0;
    double vmem_bytes_per_clk = 64.0;
    double hbm_bytes_per_s = 8.0e12 * 0.85;              // sustained fraction
    double cu_stream_bytes_per_clk = 48.0;               // one CU pulling from HBM
    int lds_per_cu = 160 * 1024;
    // split-K: fp32 partial stores per CU, and the reduce kernel's launch gap
    // and streaming rate (partials are read back from the Infinity Cache)
    double partial_store_bytes_per_us_cu = 64.0 * 2.1e3;
    double reduce_launch_us = 3.0;
    double reduce_bytes_per_us = 6.0e6;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int align8(int v) { return (v + 7) / 8 * 8; }

struct Cand {
    gemm_tile t;
    double us;
    bool screened;  // fails the padding screen
};

// Sustained MFMA issue rate of an atom relative to the dense peak, measured
// on MI355X with independent accumulators in VGPRs: the 16 x 16 x 32 bf16
// MFMA issues at about 0.57 of the peak there, the others at about 0.98.
double atom_rate(int dt, int atom)
{
    if (dt == GEMM_BF16 && atom == 16)
        return 0.57;
    return 0.98;
}

void fill_common(gemm_tile& t, int kernel, int tm, int tn, int dt, int waves = 4, int atom = 16,
                 int stages = 0, int ktb = 128)
{
    memset(&t, 0, sizeof t);
    t.kernel = kernel;
    t.tile_m = tm;
    t.tile_n = tn;
    t.tile_k = kernel == GEMM_KERNEL_SKINNY ? 0 : ktb / (dt == GEMM_BF16 ? 2 : 1);
    t.atom = atom;
    t.waves = waves;
    t.k_split = kernel == GEMM_KERNEL_SKINNY ? 4 : 1;
    t.lds_stages = stages;
}

bool price_tiled(int64_t M, int64_t N, int64_t K, int dt, int cus, int idx, const TiledRung& r, int split,
                 const Chip& c, Cand& out)
{
    const int tm = r.tm, tn = r.tn, waves = r.waves;
    if (dt == GEMM_FP8_E4M3 && r.atom == 16 && r.ktb != 128)
        return false;
    const int lds = tiled_lds_bytes(idx);
    const int vgpr = tiled_vgpr_estimate(r);
    if (lds < 0 || lds > c.lds_per_cu || vgpr > 512)
        return false;
    const int waves_per_simd = std::min(8, 512 / align8(vgpr));
    // workgroups per CU: each puts waves/4 waves on every SIMD
    const int occ = std::max(1, std::min(waves_per_simd / (waves / 4), c.lds_per_cu / lds));
    const int e = dt == GEMM_BF16 ? 2 : 1;
    const int64_t nkt = cdiv(K * e, 128);
    const int64_t tiles_m = cdiv(M, tm), tiles_n = cdiv(N, tn);
    const int64_t tiles = tiles_m * tiles_n * split;
    const double flop_tile_kt = 2.0 * tm * tn * (128.0 / e);
    const double mfma = flop_tile_kt / (c.mfma_flop_per_clk_cu[dt] * atom_rate(dt, r.atom));
    // every wave reads its rows of A from LDS once per k-tile (the 4 wave
    // columns share rows); B is read by every wave row
    const double ldsc = (4.0 * tm * 128) / c.lds_bytes_per_clk;
    const double vmem = (double)(tm + tn * (waves / 4)) * 128 / c.vmem_bytes_per_clk;
    const double per_kt = std::max(mfma, std::max(ldsc, vmem)) * (1.0 + 0.25 / occ);
    const double epi = (double)tm * tn * 2 / c.vmem_bytes_per_clk + 600.0;
    const double tile_cyc = nkt * per_kt + epi + 800.0;
    const int64_t per_cu = cdiv(tiles, cus);
    double us = per_cu * tile_cyc / c.clock_hz * 1e6;
    const double bytes = (double)M * K * e + (double)N * K * e + 2.0 * M * N;
    us = std::max(us, bytes / c.hbm_bytes_per_s * 1e6) + 2.0;
    us = calibrated_us(dt, GEMM_KERNEL_TILED, tm, tn, waves, r.atom, r.st, r.ktb, M, N, K, cus, us,
                       split);
    fill_common(out.t, GEMM_KERNEL_TILED, tm, tn, dt, waves, r.atom, r.st, r.ktb);
    const double te = (double)M * N / ((double)tiles_m * tm * (double)tiles_n * tn);
    const int64_t rounds = cdiv(tiles, cus);
    out.t.tile_eff = (float)te;
    out.t.wq_eff = (float)((double)tiles / ((double)rounds * cus));
    out.t.predicted_us = (float)us;
    out.us = us;
    out.screened = 1.0 / te > 1.25;
    return true;
}

// A and B staged in LDS: each k-tile enters the workgroup once; waves read
// their A and B fragments from LDS.
bool price_ab(int64_t M, int64_t N, int64_t K, int dt, int cus, int idx, const ABRung& r, int split,
              const Chip& c, Cand& out)
{
    const int waves = r.wm * r.wn;
    if (dt == GEMM_FP8_E4M3 && r.atom == 16 && r.ktb != 128)
        return false;
    const int lds = ab_lds_bytes(idx);
    if (lds < 0 || lds > c.lds_per_cu)
        return false;
    // accumulators + two sets of fragments + addresses
    const int acc = r.tm * r.tn / (waves * 64);
    const int frag = 2 * (r.tm / r.wm + r.tn / r.wn) / r.atom * 4 * (dt == GEMM_BF16 ? 1 : 2);
    const int vgpr = acc + frag + 40;
    const int waves_per_simd = std::min(8, 512 / align8(vgpr));
    const int occ = std::max(1, std::min(waves_per_simd / std::max(1, waves / 4), c.lds_per_cu / lds));
    const int e = dt == GEMM_BF16 ? 2 : 1;
    const int64_t nkt = cdiv(K * e, 128);
    const int64_t tiles_m = cdiv(M, r.tm), tiles_n = cdiv(N, r.tn);
    const int64_t tiles = tiles_m * tiles_n * split;
    const double flop_tile_kt = 2.0 * r.tm * r.tn * (128.0 / e);
    const double mfma = flop_tile_kt / (c.mfma_flop_per_clk_cu[dt] * atom_rate(dt, r.atom));
    const double ldsc = ((double)r.wn * r.tm * 128 + (double)r.wm * r.tn * 128) / c.lds_bytes_per_clk;
    const double vmem = (double)(r.tm + r.tn) * 128 / c.vmem_bytes_per_clk;
    const double per_kt = std::max(mfma, std::max(ldsc, vmem)) * (1.0 + 0.25 / occ);
    const double epi = (double)r.tm * r.tn * 2 / c.vmem_bytes_per_clk + 600.0;
    const double tile_cyc = nkt * per_kt + epi + 800.0;
    const int64_t per_cu = cdiv(tiles, cus);
    double us = per_cu * tile_cyc / c.clock_hz * 1e6;
    const double bytes = (double)M * K * e + (double)N * K * e + 2.0 * M * N;
    us = std::max(us, bytes / c.hbm_bytes_per_s * 1e6) + 2.0;
    us = calibrated_us(dt, GEMM_KERNEL_TILED_AB, r.tm, r.tn, waves, r.atom, r.st, r.ktb, M, N, K,
                       cus, us, split);
    fill_common(out.t, GEMM_KERNEL_TILED_AB, r.tm, r.tn, dt, waves, r.atom, r.st, r.ktb);
    const double te = (double)M * N / ((double)tiles_m * r.tm * (double)tiles_n * r.tn);
    const int64_t rounds = cdiv(tiles, cus);
    out.t.tile_eff = (float)te;
    out.t.wq_eff = (float)((double)tiles / ((double)rounds * cus));
    out.t.predicted_us = (float)us;
    out.us = us;
    out.screened = 1.0 / te > 1.25;
    return true;
}

// Ping-pong rungs: the A+B model with the 2 x 4 wave grid, unless calibrated.
bool price_pp(int64_t M, int64_t N, int64_t K, int dt, int cus, int idx, const PPRung& r, int split,
              const Chip& c, Cand& out)
{
    const int lds = pp_lds_bytes(idx);
    if (lds < 0 || lds > c.lds_per_cu)
        return false;
    const int e = dt == GEMM_BF16 ? 2 : 1;
    const int64_t nkt = cdiv(K * e, r.ktb);
    const int64_t tiles_m = cdiv(M, r.tm), tiles_n = cdiv(N, r.tn);
    const int64_t tiles = tiles_m * tiles_n * split;
    const double mfma = 2.0 * r.tm * r.tn * ((double)r.ktb / e) / (c.mfma_flop_per_clk_cu[dt] * 0.98);
    const double vmem = (double)(r.tm + r.tn) * r.ktb / c.vmem_bytes_per_clk;
    const double per_kt = std::max(mfma, vmem) * 1.25;
    const double tile_cyc = nkt * per_kt + (double)r.tm * r.tn * 2 / c.vmem_bytes_per_clk + 1400.0;
    const int64_t per_cu = cdiv(tiles, cus);
    double us = per_cu * tile_cyc / c.clock_hz * 1e6;
    const double bytes = (double)M * K * e + (double)N * K * e + 2.0 * M * N;
    us = std::max(us, bytes / c.hbm_bytes_per_s * 1e6) + 2.0;
    // An uncalibrated ping-pong rung is only ever run when forced.
    if (!find_calib(dt, GEMM_KERNEL_TILED_PP, r.tm, r.tn, 8, r.atom, r.st, r.ktb))
        return false;
    us = calibrated_us(dt, GEMM_KERNEL_TILED_PP, r.tm, r.tn, 8, r.atom, r.st, r.ktb, M, N, K, cus,
                       us, split);
    fill_common(out.t, GEMM_KERNEL_TILED_PP, r.tm, r.tn, dt, 8, r.atom, r.st, r.ktb);
    const double te = (double)M * N / ((double)tiles_m * r.tm * (double)tiles_n * r.tn);
    const int64_t rounds = cdiv(tiles, cus);
    out.t.tile_eff = (float)te;
    out.t.wq_eff = (float)((double)tiles / ((double)rounds * cus));
    out.t.predicted_us = (float)us;
    out.us = us;
    out.screened = 1.0 / te > 1.25;
    return true;
}

bool price_skinny(int64_t M, int64_t N, int64_t K, int dt, int cus, const SkinnyRung& r,
                  const Chip& c, Cand& out)
{
    const int tm = r.tm, tn = r.tn;
    if (M > tm || tm - M >= 16)
        return false;  // the smallest 16-row multiple that covers M
    const int e = dt == GEMM_BF16 ? 2 : 1;
    const int64_t nblk = cdiv(N, 16);
    const int nb = tn / 16;
    const int64_t nwg = cdiv(nblk, nb);
    const double b_bytes = (double)nblk * 16 * K * e;
    const double hbm = (b_bytes + (double)M * K * e + 2.0 * M * N);
    const double fill = std::min(1.0, (double)nwg / cus);
    double us = hbm / (c.hbm_bytes_per_s * fill) * 1e6;
    const int64_t per_cu = cdiv(nwg, cus);
    const double cu_bytes = per_cu * ((double)nb * 16 * K * e + (double)tm * K * e);
    us = std::max(us, cu_bytes / (c.cu_stream_bytes_per_clk * c.clock_hz) * 1e6) + 3.0;
    for (const SkinnyCalib& k : kSkinnyCalib)
        if (k.dt == dt && k.tm == tm && k.tn == tn && k.waves == r.waves) {
            const double wg_mb = ((double)tn * K * e + (double)tm * K * e) / 1e6;
            us = k.a * per_cu * wg_mb + k.b * hbm / 1e6 + k.c;
            break;
        }
    fill_common(out.t, GEMM_KERNEL_SKINNY, tm, tn, dt, r.waves);
    out.t.k_split = r.waves;
    const double te = (double)M * N / ((double)tm * (double)nwg * tn);
    out.t.tile_eff = (float)te;
    const int64_t rounds = cdiv(nwg, cus);
    out.t.wq_eff = (float)((double)nwg / ((double)rounds * cus));
    out.t.predicted_us = (float)us;
    out.us = us;
    out.screened = false;
    return true;
}

// Split-K costs on top of the rung's own time for one slice of K: every
// workgroup stores its fp32 partial tile, and the reduce kernel reads all
// partial planes and writes C.
double split_overhead_us(int64_t M, int64_t N, int tm, int tn, int64_t units, int S, int cus,
                         const Chip& c)
{
    const double partial = (double)cdiv(units, cus) * tm * tn * 4;
    const double reduced = (double)S * M * (double)(cdiv(N, 4) * 4) * 4 + 2.0 * M * N;
    if (kSplitCalib.points > 0)
        return kSplitCalib.d * partial / 1e6 + kSplitCalib.r1 * reduced / 1e6 + kSplitCalib.r0;
    return partial / c.partial_store_bytes_per_us_cu + c.reduce_launch_us +
           reduced / c.reduce_bytes_per_us;
}

}  // namespace

SplitPlan split_plan(int64_t M, int64_t N, int64_t K, int e, int ktb, int k_split)
{
    SplitPlan pl{1, 0, (int)(cdiv(N, 4) * 4), 0};
    const int64_t nkt = cdiv(K * e, ktb);
    const int64_t want = std::max<int64_t>(1, std::min<int64_t>(k_split, nkt));
    pl.kt_per = (int)cdiv(nkt, want);
    pl.S = (int)cdiv(nkt, pl.kt_per);
    pl.ws_bytes = pl.S > 1 ? (int64_t)pl.S * M * pl.ldw * 4 : 0;
    return pl;
}

int rung_ktb(int kernel, int idx)
{
    if (idx < 0)
        return 0;
    if (kernel == GEMM_KERNEL_TILED && idx < (int)(sizeof kTiledLadder / sizeof kTiledLadder[0]))
        return kTiledLadder[idx].ktb;
    if (kernel == GEMM_KERNEL_TILED_AB && idx < (int)(sizeof kABLadder / sizeof kABLadder[0]))
        return kABLadder[idx].ktb;
    if (kernel == GEMM_KERNEL_TILED_PP && idx < (int)(sizeof kPPLadder / sizeof kPPLadder[0]))
        return kPPLadder[idx].ktb;
    return 0;
}

int tiled_vgpr_estimate(const TiledRung& r)
{
    const int acc = r.tm * r.tn / (r.waves * 64);         // fp32 accumulators per lane
    const int b = r.tn * r.ktb / 4096 * 4 * r.st;          // B k-tiles in flight
    const int a_frag = 8;
    const int misc = 40;                      // addresses, offsets, loop state
    return acc + b + a_frag + misc;
}

int tiled_rung(int tm, int tn, int waves, int atom, int st, int ktb)
{
    int i = 0;
    for (const TiledRung& r : kTiledLadder) {
        if (r.tm == tm && r.tn == tn && r.waves == waves && r.atom == atom && DG_MATCH(r.st, r.ktb))
            return i;
        ++i;
    }
    return -1;
}

int pp_rung(int tm, int tn, int waves, int atom, int st, int ktb)
{
    if (waves != 0 && waves != 8)
        return -1;
    int i = 0;
    for (const PPRung& r : kPPLadder) {
        if (r.tm == tm && r.tn == tn && r.atom == atom && DG_MATCH(r.st, r.ktb))
            return i;
        ++i;
    }
    return -1;
}

int ab_rung(int tm, int tn, int waves, int atom, int st, int ktb)
{
    int i = 0;
    for (const ABRung& r : kABLadder) {
        if (r.tm == tm && r.tn == tn && r.wm * r.wn == waves && r.atom == atom &&
            DG_MATCH(r.st, r.ktb))
            return i;
        ++i;
    }
    return -1;
}

bool skinny_supported(int tm, int tn, int waves)
{
    for (const SkinnyRung& r : kSkinnyLadder)
        if (r.tm == tm && r.tn == tn && r.waves == waves)
            return true;
    return false;
}

// Pick the fastest candidate under the model; fill `out`.  With a workspace
// of ws_bytes, split-K variants of the tiled rungs whose partial planes fit
// are candidates too, for tiles that would leave at least half the CUs idle
// (with more, the slices add rounds instead of filling idle CUs).
void choose_tile_model(int64_t M, int64_t N, int64_t K, int dt, int cus, size_t ws_bytes,
                       gemm_tile* out);

// A shape measured on this chip (calibration.inc) gets its measured best tile
// when the device has the CU count the sweep ran on and the workspace covers
// it; any other shape is priced by the model.
void choose_tile_uncached(int64_t M, int64_t N, int64_t K, int dt, int cus, size_t ws_bytes,
                          gemm_tile* out)
{
    if (cus == 256) {
        const int e = dt == GEMM_BF16 ? 2 : 1;
        for (const MeasuredBest& b : kMeasuredBest) {
            if (b.dt != dt || b.M != M || b.N != N || b.K != K)
                continue;
            gemm_tile t;
            memset(&t, 0, sizeof t);
            t.kernel = b.kernel;
            t.tile_m = b.tm;
            t.tile_n = b.tn;
            t.tile_k = b.tile_k;
            t.atom = b.atom;
            t.waves = b.waves;
            t.k_split = b.k_split;
            t.lds_stages = b.stages;
            if (b.kernel != GEMM_KERNEL_SKINNY && b.k_split > 1) {
                int ktb = 0;
                const int idx = b.kernel == GEMM_KERNEL_TILED_AB   ? ab_rung(b.tm, b.tn, b.waves, b.atom, b.stages, b.tile_k * e)
                                : b.kernel == GEMM_KERNEL_TILED_PP ? pp_rung(b.tm, b.tn, b.waves, b.atom, b.stages, b.tile_k * e)
                                                                   : tiled_rung(b.tm, b.tn, b.waves, b.atom, b.stages, b.tile_k * e);
                ktb = rung_ktb(b.kernel, idx);
                if (ktb == 0 || split_plan(M, N, K, e, ktb, b.k_split).ws_bytes > (int64_t)ws_bytes)
                    break;   // the measured best needs more workspace: use the model
            }
            const int64_t tiles_m = cdiv(M, b.tm), tiles_n = cdiv(N, b.tn);
            const int64_t units = b.kernel == GEMM_KERNEL_SKINNY ? cdiv(cdiv(N, 16), b.tn / 16)
                                                                 : tiles_m * tiles_n * std::max(1, b.k_split);
            t.tile_eff = b.kernel == GEMM_KERNEL_SKINNY
                             ? (float)((double)M * N / ((double)b.tm * units * b.tn))
                             : (float)((double)M * N / ((double)tiles_m * b.tm * (double)tiles_n * b.tn));
            t.wq_eff = (float)((double)units / ((double)cdiv(units, cus) * cus));
            t.predicted_us = b.us;
            *out = t;
            return;
        }
    }
    choose_tile_model(M, N, K, dt, cus, ws_bytes, out);
}

void choose_tile_model(int64_t M, int64_t N, int64_t K, int dt, int cus, size_t ws_bytes,
                       gemm_tile* out)
{
    const Chip chip;
    Cand best{}, best_screened{};
    bool have = false, have_screened = false;
    auto consider = [&](const Cand& cd) {
        Cand& slot = cd.screened ? best_screened : best;
        bool& h = cd.screened ? have_screened : have;
        if (!h || cd.us < slot.us) {
            slot = cd;
            h = true;
        }
    };
    if (M <= 64) {
        for (const SkinnyRung& r : kSkinnyLadder) {
            Cand cd;
            if (price_skinny(M, N, K, dt, cus, r, chip, cd))
                consider(cd);
        }
    }
    const int e = dt == GEMM_BF16 ? 2 : 1;
    static const int kSplits[] = {1, 2, 3, 4, 6, 8, 12, 16};
    // one rung at every slice count: price(K of a slice, slices, candidate)
    auto rung = [&](int tm, int tn, int ktb, auto price) {
        for (int S : kSplits) {
            const SplitPlan pl = split_plan(M, N, K, e, ktb, S);
            if (S > 1) {
                if (ws_bytes == 0 || pl.S != S || pl.kt_per < 2 ||
                    2 * cdiv(M, tm) * cdiv(N, tn) > cus || pl.ws_bytes > (int64_t)ws_bytes ||
                    !partial_plane_fits(M, pl.ldw))
                    continue;
            }
            Cand cd;
            const int64_t Ks = S > 1 ? (int64_t)pl.kt_per * ktb / e : K;
            if (!price(Ks, S, cd))
                continue;
            if (S > 1) {
                const int64_t units = cdiv(M, tm) * cdiv(N, tn) * S;
                const double bytes = (double)M * K * e + (double)N * K * e + 2.0 * M * N;
                cd.us = std::max(cd.us + split_overhead_us(M, N, tm, tn, units, S, cus, chip),
                                 bytes / chip.hbm_bytes_per_s * 1e6);
                cd.t.k_split = S;
                cd.t.predicted_us = (float)cd.us;
            }
            consider(cd);
        }
    };
    int idx = 0;
    for (const TiledRung& r : kTiledLadder) {
        const int i = idx++;
        rung(r.tm, r.tn, r.ktb, [&](int64_t Ks, int S, Cand& cd) {
            return price_tiled(M, N, Ks, dt, cus, i, r, S, chip, cd);
        });
    }
    idx = 0;
    for (const ABRung& r : kABLadder) {
        const int i = idx++;
        rung(r.tm, r.tn, r.ktb, [&](int64_t Ks, int S, Cand& cd) {
            return price_ab(M, N, Ks, dt, cus, i, r, S, chip, cd);
        });
    }
    idx = 0;
    for (const PPRung& r : kPPLadder) {
        const int i = idx++;
        rung(r.tm, r.tn, r.ktb, [&](int64_t Ks, int S, Cand& cd) {
            return price_pp(M, N, Ks, dt, cus, i, r, S, chip, cd);
        });
    }
    *out = have ? best.t : best_screened.t;
}

// The choice is a pure function of its arguments, so it is kept per
// (M, N, K, dtype, CUs, workspace bytes): pricing the ladder costs several
// microseconds of host time, as long as a decode kernel runs.  At most
// kCacheMax shapes are kept (the table is emptied when it fills).
namespace {
struct ShapeKey {
    int64_t M, N, K;
    int dt, cus;
    size_t ws;
    bool operator==(const ShapeKey& o) const
    {
        return M == o.M && N == o.N && K == o.K && dt == o.dt && cus == o.cus && ws == o.ws;
    }
};
struct ShapeHash {
    size_t operator()(const ShapeKey& k) const
    {
        uint64_t h = 1469598103934665603ull;   // FNV-1a over the fields
        const uint64_t f[6] = {(uint64_t)k.M, (uint64_t)k.N, (uint64_t)k.K, (uint64_t)k.dt,
                               (uint64_t)k.cus, (uint64_t)k.ws};
        for (uint64_t v : f)
            h = (h ^ v) * 1099511628211ull;
        return (size_t)h;
    }
};
constexpr size_t kCacheMax = 4096;
std::mutex g_cache_mu;
std::unordered_map<ShapeKey, gemm_tile, ShapeHash> g_cache;
}  // namespace

void choose_tile(int64_t M, int64_t N, int64_t K, int dt, int cus, size_t ws_bytes, gemm_tile* out)
{
    const ShapeKey key{M, N, K, dt, cus, ws_bytes};
    {
        std::lock_guard<std::mutex> lock(g_cache_mu);
        auto it = g_cache.find(key);
        if (it != g_cache.end()) {
            *out = it->second;
            return;
        }
    }
    choose_tile_uncached(M, N, K, dt, cus, ws_bytes, out);
    std::lock_guard<std::mutex> lock(g_cache_mu);
    if (g_cache.size() >= kCacheMax)
        g_cache.clear();
    g_cache.emplace(key, *out);
}

}  // namespace dg

extern "C" gemm_status select_tile_ws(int64_t M, int64_t N, int64_t K, gemm_dtype dtype,
                                      int32_t num_cus, size_t workspace_bytes, gemm_tile* out)
{
    if (!out || M < 0 || N < 0 || K < 0 || (dtype != GEMM_BF16 && dtype != GEMM_FP8_E4M3) ||
        num_cus < 0)
        return GEMM_ERR_INVALID_VALUE;
    if (num_cus == 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return GEMM_ERR_HIP;
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            return GEMM_ERR_HIP;
        num_cus = cus;
    }
    dg::choose_tile(std::max<int64_t>(M, 1), std::max<int64_t>(N, 1), std::max<int64_t>(K, 1),
                    (int)dtype, num_cus, workspace_bytes, out);
    return GEMM_OK;
}

extern "C" gemm_status select_tile(int64_t M, int64_t N, int64_t K, gemm_dtype dtype,
                                   int32_t num_cus, gemm_tile* out)
{
    return select_tile_ws(M, N, K, dtype, num_cus, 0, out);
}
