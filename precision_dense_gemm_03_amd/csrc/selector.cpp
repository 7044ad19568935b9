// Shape -> kernel configuration selector (host only; makes no HIP call).
//
// "HGEMM优化：深度学习中的矩阵乘法性能提升策略" (jsqmd.com news 710660) §3.1 picks
// the tile from M, N and K instead of one fixed tile, and §1.1 separates small,
// medium and large problems; "DeepGEMM实战：FP8矩阵乘法与JIT编译优化指南" §3.3 picks a
// smaller tile when the edge tile would be mostly padding (M = 65 on a 64 tile)
// and §5.2 allows a manual override of the tile choice. On MI355X the rules are
// re-derived for 256 compute units:
//   1. M <= 4 (decode): the HBM-streaming kernel sized for the smallest
//      compiled M bound >= M. From M = 8 the 64x64 MFMA tile reads the
//      weight faster (FP16 [M,4096] x [4096,12288], cold weight: M = 8 52.9 us
//      vs 58.9 us streaming, M = 16 53.1 vs 109.5 us; M = 4 streams in 31.8
//      vs 52.9 us). The M = 8 and M = 16 streaming configurations stay
//      selectable by name.
//   2. Otherwise the MFMA tile kernel: the largest square tile (256, 128, 64)
//      whose grid still gives every CU a tile (>= 256 tiles; 256x256 tiles
//      from 192) and whose padded area wastes at most 25 %; if none fills the
//      chip, the tile with the most tiles (64). Which kernel runs a 256x256
//      tile is chosen in tile_with below.
//   3. LIBGEMM_CONFIG=<config name> replaces the choice when that config can
//      serve the request (same operand kind and FP8 operand formats; streaming
//      configs need M <= bound).
//   Every rule only considers configurations compiled for the requested FP8
//   operand formats (E4M3 / E5M2 for A and for B).
// Split-K plan (workspace entry points): for M <= 256 (with N = K = 4096 that
// is the HBM-bound side of the FP8 ridge point, about 600 flop per byte), when
// the chosen configuration's grid has fewer than two workgroups per CU, so
// too few loads are in flight to stream B at HBM speed, K is cut into 2, 4, 8, ...
// ranges (multiples of the configuration's K granularity) until the grid
// reaches that, or K runs out. Decode shapes are split over 64x64 tiles
// (below). LIBGEMM_SPLITS=<n> forces the number of ranges (clamped to what K
// allows).
#include <cstdlib>
#include <cstring>

#include "kernels.h"

namespace libgemm {

namespace {

constexpr int64_t kNumCUs = 256;
constexpr int64_t kStreamMaxM = 4;      // the exact mode's FP32-FMA decode kernels
// FP16 on row-major B streams only at M = 1: [M,4096]x[4096,12288] with a cold
// weight, M = 1: 21.5 us streaming against 23.1 us on the deep-ring kernel;
// M = 2 / 4: 29.8 / 31.8 us streaming against 23.3 us.
constexpr int64_t kStreamF16MaxM = 1;
constexpr int64_t kGemvMaxM = 8;        // the exact mode's FP32-FMA K-major decode kernels
// K-major B, plain calls: the dot-product decode kernels up to M = 1 (FP16) or
// M = 4 (FP8), the deep-ring kernel beyond. Cold weight, us: FP16
// [M,4096]x[4096,12288] M = 1 16.3 vs 20.7, M = 2 / 4 / 8 21.5 / 24.8 / 36.7
// vs 20.3-20.4; FP8 [M,4096]x[4096,4096] M = 4 10.7 vs 11.1, M = 8 15.6 vs 10.5.
constexpr int64_t kGemvF16MaxM = 1, kGemvFp8MaxM = 4;
constexpr int64_t kSplitMaxM = 256;
constexpr int64_t kRingMaxM = 256;

// Whether c can serve the request (operand kind, FP8 formats, B layout).
bool serves(const GemmConfig& c, int kind, int fa, int fb, int bt) {
    return c.kind == kind && serves_formats(c, fa, fb) && c.b_kmajor == bt;
}

const GemmConfig* find_named(const char* name, int kind, int64_t M, int fa = 0, int fb = 0, int bt = 0) {
    int ns = 0, nt = 0, nv = 0;
    const GemmConfig* st = stream_configs(&ns);
    const GemmConfig* tt = tile_configs(&nt);
    const GemmConfig* vt = gemv_kmajor_configs(&nv);
    for (int i = 0; i < ns; ++i)
        if (std::strcmp(st[i].name, name) == 0 && serves(st[i], kind, fa, fb, bt) && M <= st[i].bm) return &st[i];
    for (int i = 0; i < nv; ++i)
        if (std::strcmp(vt[i].name, name) == 0 && serves(vt[i], kind, fa, fb, bt) && M <= vt[i].bm) return &vt[i];
    for (int i = 0; i < nt; ++i)
        if (std::strcmp(tt[i].name, name) == 0 && serves(tt[i], kind, fa, fb, bt)) return &tt[i];
    int nd = 0;
    const GemmConfig* dt = dma_configs(&nd);
    for (int i = 0; i < nd; ++i)
        if (std::strcmp(dt[i].name, name) == 0 && serves(dt[i], kind, fa, fb, bt)) return &dt[i];
    int np = 0;
    const GemmConfig* pt = pp_configs(&np);
    for (int i = 0; i < np; ++i)
        if (std::strcmp(pt[i].name, name) == 0 && serves(pt[i], kind, fa, fb, bt)) return &pt[i];
    int nr = 0;
    const GemmConfig* rt = ring_configs(&nr);
    for (int i = 0; i < nr; ++i)
        if (std::strcmp(rt[i].name, name) == 0 && serves(rt[i], kind, fa, fb, bt)) return &rt[i];
    return nullptr;
}

// Skinny shapes (M <= 256 beyond the decode kernels): the deep-ring kernel
// whose tile minimises the bytes one compute unit must stream. A workgroup
// reads (bm + bn) K elements; a grid of more than one workgroup per compute
// unit repeats that per round. Ties go to the larger tile (fewer workgroups
// re-reading A and B).
const GemmConfig* ring_for(int kind, int64_t M, int64_t N, int fa, int fb, int bt) {
    int nr = 0;
    const GemmConfig* rt = ring_configs(&nr);
    const GemmConfig* pick = nullptr;
    int64_t best = 0;
    for (int i = 0; i < nr; ++i) {
        const GemmConfig& c = rt[i];
        if (!serves(c, kind, fa, fb, bt)) continue;
        const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
        const int64_t cost = ((tiles + kNumCUs - 1) / kNumCUs) * (c.bm + c.bn);
        if (!pick || cost < best || (cost == best && c.bm * c.bn > pick->bm * pick->bn)) {
            pick = &c;
            best = cost;
        }
    }
    return pick;
}

// The preferred configuration of each tile size. 256x256 tiles use the
// ping-pong kernel (8 waves, two per SIMD taking turns at the matrix core,
// direct loads into a 4-stage LDS ring), in its 192-row form when that leaves
// each CU fewer rows to compute: ceil(tiles / CUs) rounds of BM rows (E4M3
// 3000x4096x4096: 12 x 16 = 192 tiles of 256 rows, one round of 256, against
// 16 x 16 = 256 tiles of 192 rows, one round of 192). Smaller tiles use the
// register-staged kernel with 4 waves.
const GemmConfig* tile_with(int kind, int bm, int64_t M, int64_t N, int fa, int fb, int bt = 0) {
    if (bm == 256) {
        const int64_t tn = (N + 255) / 256;
        const int64_t rows256 = (((M + 255) / 256) * tn + kNumCUs - 1) / kNumCUs * 256;
        const int64_t rows192 = (((M + 191) / 192) * tn + kNumCUs - 1) / kNumCUs * 192;
        const bool r192 = rows192 < rows256;
        const char* want = kind == KIND_FP8
                               ? (bt ? (r192 ? "pp_fp8_192x256x64_bt" : "pp_fp8_256x256x64_bt")
                                     : (r192 ? "pp_fp8_192x256x64" : "pp_fp8_256x256x64"))
                               : (bt ? (r192 ? "pp_f16_192x256x32_bt" : "pp_f16_256x256x32_bt")
                                     : (r192 ? "pp_f16_192x256x32" : "pp_f16_256x256x32"));
        if (const GemmConfig* c = find_named(want, kind, 0, fa, fb, bt)) return c;
    }
    int nt = 0;
    const GemmConfig* tt = tile_configs(&nt);
    for (int i = 0; i < nt; ++i)
        if (serves(tt[i], kind, fa, fb, bt) && tt[i].bm == bm) return &tt[i];
    return nullptr;
}

}  // namespace

const GemmConfig* select_config(int kind, int out_dtype, int64_t M, int64_t N, int64_t K, int fa, int fb, int bt) {
    (void)out_dtype;
    (void)K;
    if (kind == KIND_F16) fa = fb = 0;
    if (const char* env = std::getenv("LIBGEMM_CONFIG")) {
        if (const GemmConfig* c = find_named(env, kind, M, fa, fb, bt)) return c;
    }
    if (bt) {
        // K-major B: decode shapes read each weight row once as a dot product
        // (no transposition, no split of K across workgroups); the first table
        // entry of the smallest bound >= M is taken.
        if (M <= (kind == KIND_F16 ? kGemvF16MaxM : kGemvFp8MaxM)) {
            int nv = 0;
            const GemmConfig* vt = gemv_kmajor_configs(&nv);
            const GemmConfig* best = nullptr;
            for (int i = 0; i < nv; ++i)
                if (serves(vt[i], kind, fa, fb, 1) && M <= vt[i].bm && (!best || vt[i].bm < best->bm)) best = &vt[i];
            if (best) return best;
        }
        if (M <= kRingMaxM) {
            if (const GemmConfig* c = ring_for(kind, M, N, fa, fb, 1)) return c;
        }
        // Tiles as for row-major B.
        static const int bt_sizes[] = {256, 128, 64};
        for (int bm : bt_sizes) {
            const int64_t tm = (M + bm - 1) / bm, tn = (N + bm - 1) / bm;
            const double useful = (double)M * (double)N;
            const double padded = (double)(tm * bm) * (double)(tn * bm);
            const int64_t min_tiles = bm == 256 ? kNumCUs * 3 / 4 : kNumCUs;
            if (tm * tn >= min_tiles && useful >= 0.75 * padded) {
                if (const GemmConfig* c = tile_with(kind, bm, M, N, fa, fb, 1)) return c;
            }
        }
        return tile_with(kind, 64, M, N, fa, fb, 1);
    }
    // The FP16 M = 1 decode streams B once through FMA sums; larger M and FP8
    // take the deep-ring kernel below (E4M3 [1,4096]x[4096,4096], cold weight:
    // 17.2 us against 19.3 us streaming).
    if (M <= kStreamF16MaxM && kind == KIND_F16) {
        const GemmConfig* best = nullptr;
        int ns = 0;
        const GemmConfig* st = stream_configs(&ns);
        for (int i = 0; i < ns; ++i) {
            const GemmConfig& c = st[i];
            if (serves(c, kind, fa, fb, 0) && M <= c.bm && (!best || c.bm < best->bm)) best = &c;
        }
        if (best) return best;
    }
    if (M <= kRingMaxM) {
        if (const GemmConfig* c = ring_for(kind, M, N, fa, fb, 0)) return c;
    }
    // 256x256 tiles already from 3/4 of the CUs (E4M3 3000x4096x4096: 61.3 us
    // on 192 ping-pong tiles vs 72.7 us on 768 tiles of 128x128).
    static const int sizes[] = {256, 128, 64};
    for (int bm : sizes) {
        const int64_t tm = (M + bm - 1) / bm, tn = (N + bm - 1) / bm;
        const double useful = (double)M * (double)N;
        const double padded = (double)(tm * bm) * (double)(tn * bm);
        const int64_t min_tiles = bm == 256 ? kNumCUs * 3 / 4 : kNumCUs;
        if (tm * tn >= min_tiles && useful >= 0.75 * padded) {
            if (const GemmConfig* c = tile_with(kind, bm, M, N, fa, fb)) return c;
        }
    }
    return tile_with(kind, 64, M, N, fa, fb);
}

const GemmConfig* select_config_exact(int out_dtype, int64_t M, int64_t N, int64_t K, int fa, int fb, int bt) {
    (void)out_dtype;
    (void)K;
    int ne = 0;
    const GemmConfig* et = exact_configs(&ne);
    if (const char* env = std::getenv("LIBGEMM_CONFIG")) {
        for (int i = 0; i < ne; ++i)
            if (std::strcmp(et[i].name, env) == 0 && serves(et[i], KIND_FP8, fa, fb, bt)) return &et[i];
        // the FP32-FMA decode kernels are exact too
        if (const GemmConfig* c = find_named(env, KIND_FP8, M, fa, fb, bt))
            if (c->family == 1 || c->family == 3) return c;
    }
    if (M <= (bt ? kGemvMaxM : kStreamMaxM)) {
        const GemmConfig* best = nullptr;
        int n = 0;
        const GemmConfig* t = bt ? gemv_kmajor_configs(&n) : stream_configs(&n);
        for (int i = 0; i < n; ++i)
            if (serves(t[i], KIND_FP8, fa, fb, bt) && M <= t[i].bm && (!best || t[i].bm < best->bm)) best = &t[i];
        if (best) return best;
    }
    auto exact_tile = [&](int bm) -> const GemmConfig* {
        for (int i = 0; i < ne; ++i)
            if (serves(et[i], KIND_FP8, fa, fb, bt) && et[i].bm == bm) return &et[i];
        return nullptr;
    };
    static const int sizes[] = {256, 128, 64};
    for (int bm : sizes) {
        const int64_t tm = (M + bm - 1) / bm, tn = (N + bm - 1) / bm;
        const double useful = (double)M * (double)N;
        const double padded = (double)(tm * bm) * (double)(tn * bm);
        const int64_t min_tiles = bm == 256 ? kNumCUs * 3 / 4 : kNumCUs;
        if (tm * tn >= min_tiles && useful >= 0.75 * padded)
            if (const GemmConfig* c = exact_tile(bm)) return c;
    }
    return exact_tile(64);
}

SplitPlan plan_splitk(int kind, int out_dtype, int64_t M, int64_t N, int64_t K, int fa, int fb, int bt) {
    if (kind == KIND_F16) fa = fb = 0;
    SplitPlan p{select_config(kind, out_dtype, M, N, K, fa, fb, bt), 1, K};
    const GemmConfig* c = p.cfg;
    if (!c || M <= 0 || N <= 0 || K <= 0 || M > kSplitMaxM) return p;
    // K-major B: decode shapes keep their dot-product kernels (each weight
    // row read once, no partial sums); larger M splits like row-major B.
    if (bt && c->family == 3) return p;
    // FP8 with row-major B up to M = 64: the deep-ring kernel's plain call is
    // replaced by split 64x64 tiles when a workspace is given (cold weight,
    // N = K = 4096, E4M3: M = 16 14.2 vs 18.0 us, M = 63 15.2 vs 18.4 us; from
    // M = 65 the two are even and the ring kernel needs no workspace; FP16
    // keeps the ring kernel: [16,4096]x[4096,12288] 25.0 vs 43.1 us).
    const bool ring_small = c->family == 6 && kind == KIND_FP8 && !bt && M <= 64;
    if ((c->family == 1 || ring_small) && !std::getenv("LIBGEMM_CONFIG")) {
        // Decode shapes split over 64x64 MFMA tiles (two launches, measured
        // against the streaming kernels' own split: FP8 N = K = 4096 M = 1
        // 13.3 vs 13.7 us, M = 4 12.9 vs 16.9 us; FP16 [M,4096]x[4096,12288]
        // M = 8 23.3 us vs 53.3 us plain), except the FP16 M = 1 decode,
        // whose plain streaming kernel (21.5 us) beats every split tried.
        if (kind == KIND_F16 && M == 1) return p;
        if (const GemmConfig* t = tile_with(kind, 64, M, N, fa, fb)) c = t;
    }
    if (c->kgran <= 0) return p;
    const int64_t base = c->family == 1 ? (N + c->bn - 1) / c->bn : ((M + c->bm - 1) / c->bm) * ((N + c->bn - 1) / c->bn);
    const int64_t max_splits = K / c->kgran;
    int64_t splits = 1;
    while (base * splits < 2 * kNumCUs && splits * 2 <= max_splits && splits < 64) splits *= 2;
    if (const char* env = std::getenv("LIBGEMM_SPLITS")) {
        const int64_t want = std::atoll(env);
        if (want >= 1) splits = want < max_splits ? want : (max_splits > 1 ? max_splits : 1);
    }
    if (splits <= 1) return p;
    const int64_t per = (K + splits - 1) / splits;
    const int64_t chunk = (per + c->kgran - 1) / c->kgran * c->kgran;
    const int64_t n = (K + chunk - 1) / chunk;
    if (n <= 1 || n > 65535) return p;
    return SplitPlan{c, (int)n, chunk};
}

}  // namespace libgemm
