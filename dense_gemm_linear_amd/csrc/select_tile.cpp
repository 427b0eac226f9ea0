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

#include "internal.hpp"

namespace dg {

namespace {

// Measured per-rung cost constants (calibrate.py): t_us = a * n_cu * K_bytes
// / 1000 + b * n_cu + c, n_cu = ceil(tiles / CUs).
struct RungCalib {
    int dt, kernel, tm, tn, waves, atom, st, ktb;
    float a, b, c;
    int points;
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

// Calibrated time of a tiled / A+B rung, or `fallback` if it was never measured.
double calibrated_us(int dt, int kernel, int tm, int tn, int waves, int atom, int st, int ktb,
                     int64_t M, int64_t N, int64_t K, int cus, double fallback)
{
    const RungCalib* r = find_calib(dt, kernel, tm, tn, waves, atom, st, ktb);
    if (!r)
        return fallback;
    const int e = dt == GEMM_BF16 ? 2 : 1;
    const int64_t tiles = ((M + tm - 1) / tm) * ((N + tn - 1) / tn);
    const double ncu = (double)((tiles + cus - 1) / cus);
    return r->a * ncu * (double)K * e / 1000.0 + r->b * ncu + r->c;
}

struct Chip {
    double clock_hz = 2.4e9;
    double mfma_flop_per_clk_cu[2] = {4096.0, 8192.0};  // bf16, e4m3 dense
    double lds_bytes_per_clk = 128.0;
    double vmem_bytes_per_clk = 64.0;
    double hbm_bytes_per_s = 8.0e12 * 0.85;              // sustained fraction
    double cu_stream_bytes_per_clk = 48.0;               // one CU pulling from HBM
    int lds_per_cu = 160 * 1024;
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

bool price_tiled(int64_t M, int64_t N, int64_t K, int dt, int cus, int idx, const TiledRung& r,
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
    const int64_t tiles = tiles_m * tiles_n;
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
    us = calibrated_us(dt, GEMM_KERNEL_TILED, tm, tn, waves, r.atom, r.st, r.ktb, M, N, K, cus, us);
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
bool price_ab(int64_t M, int64_t N, int64_t K, int dt, int cus, int idx, const ABRung& r,
              const Chip& c, Cand& out)
{
    const int waves = r.wm * r.wn;
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
    const int64_t tiles = tiles_m * tiles_n;
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
                       cus, us);
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
bool price_pp(int64_t M, int64_t N, int64_t K, int dt, int cus, int idx, const PPRung& r,
              const Chip& c, Cand& out)
{
    const int lds = pp_lds_bytes(idx);
    if (lds < 0 || lds > c.lds_per_cu)
        return false;
    const int e = dt == GEMM_BF16 ? 2 : 1;
    const int64_t nkt = cdiv(K * e, r.ktb);
    const int64_t tiles_m = cdiv(M, r.tm), tiles_n = cdiv(N, r.tn);
    const int64_t tiles = tiles_m * tiles_n;
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
                       us);
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

}  // namespace

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

// Pick the fastest candidate under the model; fill `out`.
void choose_tile(int64_t M, int64_t N, int64_t K, int dt, int cus, gemm_tile* out)
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
    int idx = 0;
    for (const TiledRung& r : kTiledLadder) {
        Cand cd;
        if (price_tiled(M, N, K, dt, cus, idx++, r, chip, cd))
            consider(cd);
    }
    idx = 0;
    for (const ABRung& r : kABLadder) {
        Cand cd;
        if (price_ab(M, N, K, dt, cus, idx++, r, chip, cd))
            consider(cd);
    }
    idx = 0;
    for (const PPRung& r : kPPLadder) {
        Cand cd;
        if (price_pp(M, N, K, dt, cus, idx++, r, chip, cd))
            consider(cd);
    }
    *out = have ? best.t : best_screened.t;
}

}  // namespace dg

extern "C" gemm_status select_tile(int64_t M, int64_t N, int64_t K, gemm_dtype dtype,
                                   int32_t num_cus, gemm_tile* out)
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
                    (int)dtype, num_cus, out);
    return GEMM_OK;
}
